"""Whole-layer parity: moe_layer_fwd against the oracle's layer_forward on the same
seeded inputs, each side quantising the fp32 weights itself."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as M
import oracle as O
from oracle import codecs as OC
import synth
from gpu_util import TOL, dev, error_ratios, fp8_layer_errors, note, to_np, ulp_bf16

pytestmark = pytest.mark.gpu


def _gpu_weights(w: synth.Workload, inp: dict) -> dict:
    d = dev()
    out = {"w_router": inp.get("w_router"), "bias": inp.get("bias")}
    out = {k: (v.to(d) if v is not None else None) for k, v in out.items()}
    if w.mode == "fp32":
        out["w13"], out["w2"] = inp["w13"].to(d), inp["w2"].to(d)
    elif w.mode == "fp8":
        q13, out["s13"] = M.moe_quant_weight_fp8(inp["w13"].to(d))
        q2, out["s2"] = M.moe_quant_weight_fp8(inp["w2"].to(d))
        out["w13"], out["w2"] = M.moe_pack_weight_fp8(q13), M.moe_pack_weight_fp8(q2)
    else:
        out["w13"], out["s13"] = M.moe_quant_weight_int4(inp["w13"].to(d))
        out["w2"], out["s2"] = M.moe_quant_weight_int4(inp["w2"].to(d))
    return out


def _oracle_experts(w: synth.Workload, inp: dict):
    w13, w2 = inp["w13"].cpu().numpy(), inp["w2"].cpu().numpy()
    if w.mode == "fp32":
        return (w13, w2)
    if w.mode == "fp8":
        return (*OC.quant_fp8_weight(w13), *OC.quant_fp8_weight(w2))
    return (*OC.int4_quant_rows(w13), *OC.int4_quant_rows(w2))


def _near_ties(logits32, bias, k, margin):
    """Tokens whose k-th and (k+1)-th keys are closer than ``margin``: either choice
    is a correct routing, so their outputs are compared only through the routing check."""
    key = (logits32 + bias[None, :]).astype(np.float32).astype(np.float64)
    srt = -np.sort(-key, axis=1)
    if k >= key.shape[1]:
        return np.zeros(key.shape[0], bool)
    return (srt[:, k - 1] - srt[:, k]) < margin


def run_layer_case(w: synth.Workload, tokens=None, cap_factor=0.0):
    note(f"layer {w.name} T={w.T} d={w.d} E={w.E} k={w.k} I={w.I} mode={w.mode} "
         f"cap_factor={cap_factor}")
    inp = synth.layer_inputs(w)
    gw = _gpu_weights(w, inp)
    desc = M.LayerDesc(w.T, w.d, w.E, w.k, w.I, mode=w.mode, route=w.route, m_align=w.m_align,
                       capacity_factor=cap_factor)
    x = inp["x"].to(dev())
    ids = inp.get("token_ids")
    y, counts = M.moe_layer_fwd(desc, gw, x, ids.to(dev()) if ids is not None else None)
    torch.cuda.synchronize()
    ref = O.layer_forward(w.mode, inp["x"].float().numpy(), E=w.E, k=w.k, I=w.I,
                          m_align=w.m_align,
                          w_router=None if w.route == "hash" else inp["w_router"].float().numpy(),
                          bias=None if w.route == "hash" else inp["bias"].numpy(),
                          token_ids=None if ids is None else ids.numpy(),
                          experts=_oracle_experts(w, inp), tokens=tokens,
                          keep=(w.mode == "fp8"), cap_factor=cap_factor)
    rows = np.arange(w.T) if tokens is None else np.asarray(tokens)
    if w.route == "score":
        amb = _near_ties(ref["logits"].astype(np.float32), inp["bias"].numpy(), w.k, 1e-5)
    else:
        amb = np.zeros(w.T, bool)
    if not amb.any():
        np.testing.assert_array_equal(to_np(counts), ref["counts"])
    keep = rows[~amb[rows]]
    yg = to_np(y).astype(np.float64)[keep]
    yr = ref["y"][keep]
    if w.mode == "fp32":
        beyond, raw = error_ratios(yg, yr, rounding=0.0)
        print(f"raw={raw:.3e}")
        assert raw <= TOL
        return ref
    if w.mode == "fp8":
        e = fp8_layer_errors(yg, ref, keep, w.T, w.k)
        print(f"errors {e} ambiguous_tokens={int(amb.sum())}")
        assert e["beyond_flip"] <= TOL
        return ref
    # w4a16: bf16 output of y plus the bf16 expert rows it sums
    r = 0.5 * ulp_bf16(yr)
    wk = np.asarray(ref["w"]).reshape(w.T, w.k)
    for i, t in enumerate(keep):
        for j in range(w.k):
            s = t * w.k + j
            if s in ref["o_by_slot"]:
                r[i] += abs(wk[t, j]) * 0.5 * ulp_bf16(ref["o_by_slot"][s])
    beyond, raw = error_ratios(yg, yr, rounding=r)
    print(f"beyond={beyond:.3e} raw={raw:.3e} ambiguous={int(amb.sum())}")
    assert beyond <= TOL
    return ref


def test_layer_tiny_fp32():
    run_layer_case(synth.WORKLOADS["tiny_fp32"])


def test_layer_small_fp8():
    run_layer_case(synth.Workload("small_fp8", T=96, d=256, E=8, k=2, I=256, mode="fp8",
                                  skew_frac=0.25, skew_add=2.0, m_align=16))


def test_layer_small_fp8_many_experts():
    run_layer_case(synth.Workload("small_fp8_e64", T=200, d=384, E=64, k=6, I=128, mode="fp8",
                                  m_align=32, seed=3))


@pytest.mark.parametrize("mode", ["fp8", "fp32"])
def test_layer_capacity_drop(mode):
    """Capacity floor(ceil(T*k/E) * 1.0) with skewed routing: the favoured experts
    overflow and their late slots are dropped (contribute nothing)."""
    w = synth.Workload(f"cap_{mode}", T=96, d=256, E=8, k=2, I=256, mode=mode,
                       skew_frac=0.25, skew_add=2.0, m_align=16, seed=5)
    cap = M.moe_capacity(w.T, w.k, w.E, 1.0)
    assert cap == -(-w.T * w.k // w.E)
    ref = run_layer_case(w, cap_factor=1.0)
    dropped = int(np.maximum(np.asarray(ref["counts"]) - cap, 0).sum())
    print(f"capacity {cap}, dropped slots {dropped}")
    assert dropped > 0


def test_layer_small_w4a16_hash():
    run_layer_case(synth.Workload("small_w4a16", T=300, d=256, E=8, k=1, I=256, mode="w4a16",
                                  route="hash", m_align=64))
