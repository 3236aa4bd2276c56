"""Whole-layer parity: moe_layer_fwd against the oracle's layer_forward on the same
seeded inputs, each side quantising the fp32 weights itself."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as M
import oracle as O
from oracle import codecs as OC
import synth
from gpu_util import (TOL, check_counts_outside_ties, dev, error_ratios, fp8_layer_errors,
                      gpu_h_by_slot, note, staged_fp8_layer, to_np, ulp_bf16)

pytestmark = pytest.mark.gpu


def _gpu_weights(w: synth.Workload, inp: dict) -> dict:
    d = dev()
    out = {"w_router": inp.get("w_router"), "bias": inp.get("bias")}
    out = {k: (v.to(d) if v is not None else None) for k, v in out.items()}
    if w.mode == "fp32":
        out["w13"], out["w2"] = inp["w13"].to(d), inp["w2"].to(d)
    elif w.mode == "w4a8":
        q13, s13 = M.moe_quant_weight_int4(inp["w13"].to(d))
        q2, s2 = M.moe_quant_weight_int4(inp["w2"].to(d))
        out["w13"], out["s13"] = M.moe_pack_weight_int4(q13, s13)
        out["w2"], out["s2"] = M.moe_pack_weight_int4(q2, s2)
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
    if w.mode == "w4a8":
        return (*OC.int4_quant_rows(w13), *OC.int4_quant_rows(w2))
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


def run_layer_case(w: synth.Workload, tokens=None, cap_factor=0.0, renorm=False,
                   layout="contiguous"):
    note(f"layer {w.name} T={w.T} d={w.d} E={w.E} k={w.k} I={w.I} mode={w.mode} "
         f"cap_factor={cap_factor} renorm={renorm} layout={layout}")
    inp = synth.layer_inputs(w)
    gw = _gpu_weights(w, inp)
    desc = M.LayerDesc(w.T, w.d, w.E, w.k, w.I, mode=w.mode, route=w.route, m_align=w.m_align,
                       capacity_factor=cap_factor, renorm=renorm, layout=layout)
    x = inp["x"].to(dev())
    ids = inp.get("token_ids")
    y, counts = M.moe_layer_fwd(desc, gw, x, ids.to(dev()) if ids is not None else None)
    staged = None
    if w.mode in ("fp8", "w4a8"):
        # the same kernels through the individual entry points: bit-identical, and they
        # expose GEMM1's requantised h for the flip accounting below
        staged = staged_fp8_layer(M, w.T, w.E, w.k, w.I, w.m_align, x, gw, renorm=renorm,
                                  capacity=M.moe_capacity(w.T, w.k, w.E, cap_factor),
                                  w4a8=w.mode == "w4a8",
                                  token_ids=ids.to(dev()) if ids is not None else None)
        # (masked layout: the same expert rows at other places, so the same y bit for bit)
        assert torch.equal(staged["y"], y) and torch.equal(staged["counts"], counts)
    torch.cuda.synchronize()
    ref = O.layer_forward(w.mode, inp["x"].float().numpy(), E=w.E, k=w.k, I=w.I,
                          m_align=w.m_align,
                          w_router=None if w.route == "hash" else inp["w_router"].float().numpy(),
                          bias=None if w.route == "hash" else inp["bias"].numpy(),
                          token_ids=None if ids is None else ids.numpy(),
                          experts=_oracle_experts(w, inp), tokens=tokens,
                          keep=(w.mode in ("fp8", "w4a8")), cap_factor=cap_factor,
                          renorm=renorm)
    rows = np.arange(w.T) if tokens is None else np.asarray(tokens)
    if w.route == "score":
        amb = _near_ties(ref["logits"].astype(np.float32), inp["bias"].numpy(), w.k, 1e-5)
    else:
        amb = np.zeros(w.T, bool)
    if w.route == "score":
        n_checked = check_counts_outside_ties(to_np(counts), ref, inp["bias"].numpy(), w.k, 1e-5)
        print(f"counts checked for {n_checked} of {w.E} experts")
    else:
        np.testing.assert_array_equal(to_np(counts), ref["counts"])
    keep = rows[~amb[rows]]
    yg = to_np(y).astype(np.float64)[keep]
    yr = ref["y"][keep]
    if w.mode == "fp32":
        beyond, raw = error_ratios(yg, yr, rounding=0.0)
        print(f"raw={raw:.3e}")
        assert raw <= TOL
        return ref
    if w.mode in ("fp8", "w4a8"):
        slots = [t * w.k + j for t in keep for j in range(w.k)]
        np.testing.assert_array_equal(to_np(staged["idx"])[keep], ref["idx"][keep])
        h_gpu = gpu_h_by_slot(staged, slots)
        e = fp8_layer_errors(yg, ref, keep, w.T, w.k, h_gpu)
        print(f"errors {e} near_tie_tokens={int(amb.sum())}")
        assert e["beyond_flip"] <= TOL
        assert e["beyond_noflip"] <= TOL
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


@pytest.mark.parametrize("mode", ["fp8", "fp32"])
def test_layer_renorm(mode):
    """MOE_ROUTE_RENORM: the k gate weights divided by their sum (top-k then softmax)."""
    run_layer_case(synth.Workload(f"renorm_{mode}", T=80, d=256, E=8, k=3, I=256, mode=mode,
                                  m_align=16, seed=9), renorm=True)


def test_layer_big_tiles(monkeypatch):
    """Few large experts (about 770 rows each): with FP8GG_BIG_TILES=1 the layer's GEMM1
    (SwiGLU, 32 column tiles, so 8 row tiles a round) sends each expert's leading 256-row
    tiles to the 256 x 256-tile kernel; the layer must still match the per-step entry
    points bit for bit and the oracle on sampled tokens."""
    monkeypatch.setenv("FP8GG_BIG_TILES", "1")
    w = synth.Workload("big_tiles_fp8", T=1024, d=2048, E=4, k=3, I=4096, mode="fp8",
                       m_align=16, seed=5)
    run_layer_case(w, tokens=[0, 1, 2, 100, 511, 512, 700, 1000, 1022, 1023])


@pytest.mark.parametrize("mode", ["fp8", "fp32", "w4a16"])
def test_layer_single_token(mode):
    """Degenerate batch: one token, every one of its k experts holding a single row (the
    rest empty), k = E - 1 so that one expert is untouched."""
    route = "hash" if mode == "w4a16" else "score"
    run_layer_case(synth.Workload(f"one_{mode}", T=1, d=256, E=8, k=1 if route == "hash" else 7,
                                  I=256, mode=mode, route=route, m_align=16, seed=4))


@pytest.mark.parametrize("mode", ["fp8", "fp32"])
def test_layer_no_tokens(mode):
    """T = 0: nothing to compute, and the reported routed counts are all 0 (the output
    buffer is overwritten, whatever it held)."""
    note(f"layer T=0 mode={mode}")
    w = synth.Workload(f"empty_{mode}", T=4, d=256, E=8, k=2, I=256, mode=mode, m_align=16)
    inp = synth.layer_inputs(w)
    gw = _gpu_weights(w, inp)
    desc = M.LayerDesc(0, w.d, w.E, w.k, w.I, mode=w.mode, route=w.route, m_align=w.m_align)
    x = inp["x"][:0].to(dev())
    counts = torch.full((w.E,), -7, dtype=torch.int32, device=dev())
    y, counts = M.moe_layer_fwd(desc, gw, x, None, counts=counts)
    torch.cuda.synchronize()
    assert y.shape == (0, w.d)
    assert torch.equal(counts.cpu(), torch.zeros(w.E, dtype=torch.int32))


@pytest.mark.parametrize("E", [300, 520])
def test_layer_fp8_wide_expert_counts(E):
    """Expert counts past the 256-expert dispatch instance: the 512-expert one (its
    workgroups 1.. quantising the tokens) and the separate count/scatter launches above
    512 experts, with most experts empty."""
    run_layer_case(synth.Workload(f"wide_e{E}", T=64, d=256, E=E, k=4, I=256, mode="fp8",
                                  m_align=16, seed=6))


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


@pytest.mark.parametrize("cap_factor", [1.0, 2.0])
def test_layer_masked_layout(cap_factor):
    """Fixed-capacity layout ([E, C, d] buffers, masked GEMMs): the oracle's layer with that
    capacity, and bit for bit the contiguous layout with the same capacity."""
    w = synth.Workload("masked_fp8", T=96, d=256, E=8, k=2, I=256, mode="fp8",
                       skew_frac=0.25, skew_add=2.0, m_align=16, seed=5)
    run_layer_case(w, cap_factor=cap_factor, layout="masked")


def test_layer_small_w4a8():
    """4-bit expert weights on the FP8 matrix core, score routing."""
    run_layer_case(synth.Workload("small_w4a8", T=96, d=256, E=8, k=2, I=256, mode="w4a8",
                                  skew_frac=0.25, skew_add=2.0, m_align=16, seed=2))


def test_layer_small_w4a8_hash():
    run_layer_case(synth.Workload("small_w4a8_hash", T=300, d=256, E=8, k=1, I=256,
                                  mode="w4a8", route="hash", m_align=64))


def test_layer_small_w4a16_hash():
    run_layer_case(synth.Workload("small_w4a16", T=300, d=256, E=8, k=1, I=256, mode="w4a16",
                                  route="hash", m_align=64))


# ------------------------------------------------------------ chunked pipeline

def _near_tie_tokens(w, inp, margin):
    if w.route != "score":
        return np.zeros(w.T, bool)
    logits = O.router_logits(inp["x"].float().numpy(), inp["w_router"].float().numpy())
    return _near_ties(logits.astype(np.float32), inp["bias"].numpy(), w.k, margin)


@pytest.mark.parametrize("mode,chunk", [("fp8", 128), ("fp8", 64), ("fp32", 100)])
def test_layer_chunked_pipeline(mode, chunk):
    """Two-stream chunk pipeline: every chunk an independent layer pass (the last ragged),
    matched to the oracle's whole-batch layer."""
    w = synth.Workload(f"chunked_{mode}", T=300, d=256, E=8, k=2, I=256, mode=mode,
                       skew_frac=0.25, skew_add=2.0, m_align=16, seed=11)
    note(f"chunked layer {mode} T={w.T} chunk={chunk}")
    inp = synth.layer_inputs(w)
    gw = _gpu_weights(w, inp)
    desc = M.LayerDesc(w.T, w.d, w.E, w.k, w.I, mode=w.mode, m_align=w.m_align)
    x = inp["x"].to(dev())
    y = M.moe_layer_fwd_chunked(desc, gw, x, chunk)
    y1, _ = M.moe_layer_fwd(desc, gw, x)
    staged = staged_fp8_layer(M, w.T, w.E, w.k, w.I, w.m_align, x, gw) if mode == "fp8" else None
    torch.cuda.synchronize()
    ref = O.layer_forward(w.mode, inp["x"].float().numpy(), E=w.E, k=w.k, I=w.I,
                          m_align=w.m_align, w_router=inp["w_router"].float().numpy(),
                          bias=inp["bias"].numpy(), experts=_oracle_experts(w, inp),
                          keep=(mode == "fp8"))
    amb = _near_tie_tokens(w, inp, 1e-4)
    keep = np.nonzero(~amb)[0]
    yg = to_np(y).astype(np.float64)
    # against the single pass: the same experts' rows; only the gate weights' last bits
    # (the router's split-K order depends on the chunk size) may differ
    d1 = np.abs(yg[keep] - to_np(y1).astype(np.float64)[keep]).max()
    print(f"chunked vs single pass: max |diff| {d1:.3e}, near-tie tokens {int(amb.sum())}")
    if mode == "fp32":
        beyond, raw = error_ratios(yg[keep], ref["y"][keep], rounding=0.0)
        print(f"raw={raw:.3e}")
        assert raw <= TOL
        return
    h_gpu = gpu_h_by_slot(staged, [t * w.k + j for t in keep for j in range(w.k)])
    e = fp8_layer_errors(yg[keep], ref, keep, w.T, w.k, h_gpu)
    print(f"errors {e}")
    assert e["beyond_flip"] <= TOL and e["beyond_noflip"] <= TOL


def test_layer_chunked_pipeline_hash_bitexact():
    """Hash routing has no logits: the chunk pipeline then gives the single pass's output
    bit for bit (the same expert rows, summed in the same order)."""
    w = synth.Workload("chunked_w4a16", T=300, d=256, E=8, k=1, I=256, mode="w4a16",
                       route="hash", m_align=64)
    note(f"chunked layer w4a16 hash T={w.T} chunk=128")
    inp = synth.layer_inputs(w)
    gw = _gpu_weights(w, inp)
    desc = M.LayerDesc(w.T, w.d, w.E, w.k, w.I, mode=w.mode, route="hash", m_align=w.m_align)
    x, ids = inp["x"].to(dev()), inp["token_ids"].to(dev())
    y = M.moe_layer_fwd_chunked(desc, gw, x, 128, token_ids=ids)
    y1, _ = M.moe_layer_fwd(desc, gw, x, ids)
    torch.cuda.synchronize()
    assert torch.equal(y, y1)
