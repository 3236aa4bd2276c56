"""Parity at the workloads' full sizes, in the launch configuration the bench times.

The GPU runs the whole batch; the oracle recomputes sampled outputs one by one (a few
tokens of each layer, sampled rows x column blocks of the standalone grouped GEMM),
quantising only the expert weights those samples touch.  Integer results that are
fully checkable (routing of every token, dispatch counts) are checked in full.
"""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as M
import oracle as O
from oracle import codecs as OC
import synth
from gpu_util import (C_MFMA_FP8, TOL, dev, error_ratios, fp8_layer_errors, note, to_np,
                      ulp_bf16)

pytestmark = pytest.mark.gpu


class LazyExperts:
    """Per-expert weights quantised by the oracle on first use, from fp32 masters that
    live on the GPU (generated there by the seeded generator).  Slicing [e:e+1] returns
    that expert's codes or scales, as layer_forward expects of full arrays."""

    def __init__(self, master: torch.Tensor, kind: str):
        self.master, self.kind, self.cache = master, kind, {}

    def _get(self, e):
        if e not in self.cache:
            w = self.master[e:e + 1].float().cpu().numpy()
            self.cache[e] = (OC.quant_fp8_weight(w) if self.kind == "fp8"
                             else OC.int4_quant_rows(w))
        return self.cache[e]

    def view(self, which):
        outer = self

        class _V:
            def __getitem__(self, sl):
                assert isinstance(sl, slice) and sl.stop == sl.start + 1
                return outer._get(sl.start)[which]
        return _V()


def _layer_fullsize(w: synth.Workload, tokens):
    note(f"full-size layer {w.name} T={w.T} d={w.d} E={w.E} k={w.k} I={w.I} tokens={tokens}")
    d = dev()
    inp = synth.layer_inputs(w, device=d)
    if w.mode == "fp8":
        q13, s13 = M.moe_quant_weight_fp8(inp["w13"])
        q2, s2 = M.moe_quant_weight_fp8(inp["w2"])
    else:
        q13, s13 = M.moe_quant_weight_int4(inp["w13"])
        q2, s2 = M.moe_quant_weight_int4(inp["w2"])
    if w.mode == "fp8":
        q13, q2 = M.moe_pack_weight_fp8(q13), M.moe_pack_weight_fp8(q2)
    weights = {"w13": q13, "s13": s13, "w2": q2, "s2": s2}
    if w.route == "score":
        weights.update(w_router=inp["w_router"], bias=inp["bias"])
    desc = M.LayerDesc(w.T, w.d, w.E, w.k, w.I, mode=w.mode, route=w.route, m_align=w.m_align)
    y, counts = M.moe_layer_fwd(desc, weights, inp["x"], inp.get("token_ids"))
    torch.cuda.synchronize()
    del q13, q2
    e13, e2 = LazyExperts(inp["w13"], w.mode), LazyExperts(inp["w2"], w.mode)
    experts = (e13.view(0), e13.view(1), e2.view(0), e2.view(1))
    ids = inp.get("token_ids")
    ref = O.layer_forward(w.mode, inp["x"].float().cpu().numpy(), E=w.E, k=w.k, I=w.I,
                          m_align=w.m_align,
                          w_router=None if ids is not None else inp["w_router"].float().cpu().numpy(),
                          bias=None if ids is not None else inp["bias"].cpu().numpy(),
                          token_ids=None if ids is None else ids.cpu().numpy(),
                          experts=experts, tokens=tokens, keep=(w.mode == "fp8"))
    # routing of every token: identical unless two keys tie within the fp32 logit error
    if w.route == "score":
        key = ref["logits"].astype(np.float32) + inp["bias"].cpu().numpy()[None, :]
        srt = -np.sort(-key.astype(np.float64), axis=1)
        amb = (srt[:, w.k - 1] - srt[:, w.k]) < 1e-4
        print(f"near-tie tokens {int(amb.sum())} of {w.T}")
        if not amb.any():
            np.testing.assert_array_equal(to_np(counts), ref["counts"])
        tokens = [t for t in tokens if not amb[t]]
    else:
        np.testing.assert_array_equal(to_np(counts), ref["counts"])
    yg = to_np(y[tokens]).astype(np.float64)
    if w.mode == "fp8":
        e = fp8_layer_errors(yg, ref, np.asarray(tokens), w.T, w.k)
        print(f"errors {e}")
        assert e["beyond_flip"] <= TOL
    else:
        yr = ref["y"][tokens]
        r = 0.5 * ulp_bf16(yr)
        for i, t in enumerate(tokens):
            r[i] += 0.5 * ulp_bf16(ref["o_by_slot"][t])
        beyond, raw = error_ratios(yg, yr, rounding=r)
        print(f"beyond={beyond:.3e} raw={raw:.3e}")
        assert beyond <= TOL


def test_fullsize_prefill_layer():
    _layer_fullsize(synth.scaled(synth.WORKLOADS["prefill_fp8"], m_align=16), [0, 2049])


def test_fullsize_decode_layer():
    _layer_fullsize(synth.WORKLOADS["decode_fp8"], [5, 127])


def test_fullsize_hash_w4a16_layer():
    _layer_fullsize(synth.WORKLOADS["hash_w4a16"], [0, 1, 4096, 8191])


def test_fullsize_grouped_gemm_fp8():
    """16 groups, sizes ~ Zipf(1.1) summing to 8192, each padded to 128; N=4096, K=7168."""
    sizes = synth.zipf_group_sizes(8192, 16, 1.1, seed=0)
    N, K = 4096, 7168
    note(f"full-size grouped GEMM sizes={sizes.tolist()} N={N} K={K}")
    padded = -(-sizes // 128) * 128
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    R = int(offsets[-1])
    d = dev()
    g = synth.gemm_inputs(sizes, N, K, seed=0, device=d)
    dest = np.concatenate([np.arange(offsets[i], offsets[i] + sizes[i]) for i in range(16)])
    a = torch.zeros((R, K), dtype=torch.float32, device=d)
    a[torch.from_numpy(dest).to(d)] = g["a"]
    qa, sa = M.moe_quant_fp8(a)
    qb, sb = M.moe_quant_weight_fp8(g["b"])
    c = M.grouped_gemm_fp8(qa, sa, M.moe_pack_weight_fp8(qb), sb, torch.from_numpy(offsets).to(d),
                           R, N)
    torch.cuda.synchronize()
    rows = np.concatenate([[offsets[i], offsets[i] + sizes[i] - 1] for i in range(16)])
    cblocks = [0, 17, 31]
    cols = np.concatenate([np.arange(cb * 128, cb * 128 + 128) for cb in cblocks])
    a_s = a[torch.from_numpy(rows).to(d)].cpu().numpy()
    qao, sao = OC.quant_fp8_act(a_s)
    np.testing.assert_array_equal(to_np(qa[torch.from_numpy(rows).to(d)]), qao)
    beyond_all, raw_all, model_ok = 0.0, 0.0, True
    for gi in range(16):
        bsub = g["b"][gi:gi + 1, torch.from_numpy(cols).to(d)].cpu().numpy()
        qbo, sbo = OC.quant_fp8_weight(bsub)
        np.testing.assert_array_equal(to_np(qb[gi:gi + 1, torch.from_numpy(cols).to(d)]), qbo)
        sel = [j for j, r in enumerate(rows) if offsets[gi] <= r < offsets[gi + 1]]
        A = OC.dequant_fp8_act(qao[sel], sao[sel])
        B = OC.dequant_fp8_weight(qbo, sbo)[0]
        ref = A @ B.T
        gpu = to_np(c[torch.from_numpy(rows[sel]).to(d)][:, torch.from_numpy(cols).to(d)])
        beyond, raw = error_ratios(gpu, ref)
        beyond_all, raw_all = max(beyond_all, beyond), max(raw_all, raw)
        bound = C_MFMA_FP8 * (np.abs(A) @ np.abs(B).T) + 0.5 * ulp_bf16(ref) + 1e-30
        model_ok &= bool(np.all(np.abs(gpu - ref) <= bound * 1.0001))
    print(f"beyond={beyond_all:.3e} raw={raw_all:.3e} within MFMA error model: {model_ok}")
    assert beyond_all <= TOL
    assert model_ok
