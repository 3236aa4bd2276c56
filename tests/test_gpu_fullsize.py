"""Parity at the workloads' full sizes, in the launch configuration the bench times.

The GPU runs the whole batch; the oracle recomputes sampled outputs one by one (a few
tokens of each layer, sampled rows x column blocks of the standalone grouped GEMM),
quantising only the expert weights those samples touch.  Integer results that are
fully checkable (routing of every token, dispatch counts) are checked in full.
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as M
import oracle as O
from oracle import codecs as OC
import synth
from gpu_util import (C_MFMA_FP8, TOL, check_counts_outside_ties, dev, error_ratios,
                      fp8_layer_errors, gpu_h_by_slot, note, staged_fp8_layer, to_np,
                      ulp_bf16)

pytestmark = pytest.mark.gpu


class LazyExperts:
    """Per-expert weights quantised by the oracle on first use, from fp32 masters that
    live on the GPU (generated there by the seeded generator).  Slicing [e:e+1] returns
    that expert's codes or scales, as layer_forward expects of full arrays.  prefetch()
    quantises a set of experts on host threads (numpy releases the GIL in its array
    loops)."""

    def __init__(self, master: torch.Tensor, kind: str):
        self.master, self.kind, self.cache = master, kind, {}

    def _quant(self, w):
        return OC.quant_fp8_weight(w) if self.kind == "fp8" else OC.int4_quant_rows(w)

    def prefetch(self, experts, threads=16):
        todo = [int(e) for e in experts if int(e) not in self.cache]
        hosts = [self.master[e:e + 1].float().cpu().numpy() for e in todo]
        with cf.ThreadPoolExecutor(threads) as ex:
            for e, r in zip(todo, ex.map(self._quant, hosts)):
                self.cache[e] = r

    def _get(self, e):
        if e not in self.cache:
            self.cache[e] = self._quant(self.master[e:e + 1].float().cpu().numpy())
        return self.cache[e]

    def view(self, which):
        outer = self

        class _V:
            def __getitem__(self, sl):
                assert isinstance(sl, slice) and sl.stop == sl.start + 1
                return outer._get(sl.start)[which]
        return _V()


def _pick_tokens(idx, counts, near_tie, bms, n_tokens, max_experts):
    """Tokens for the sampled comparison: greedily the ones adding the fewest experts not
    yet covered, until ``n_tokens`` are chosen, while making sure both tile classes (groups
    of at most ``bms`` rows and larger groups) appear.  Near-tie tokens are skipped."""
    small = set(np.nonzero((counts > 0) & (counts <= bms))[0].tolist())
    cand = [t for t in range(idx.shape[0]) if not near_tie[t]]
    chosen, cover = [], set()
    need_small = 3
    while len(chosen) < n_tokens and cand:
        def cost(t):
            es = set(idx[t].tolist())
            new = len(es - cover)
            has_small = len(es & small) > 0
            return (new - (2 if (need_small > 0 and has_small and es - cover & small) else 0), t)
        t = min(cand, key=cost)
        es = set(idx[t].tolist())
        if len(cover | es) > max_experts:
            break
        if es - cover & small:
            need_small -= 1
        cover |= es
        chosen.append(t)
        cand.remove(t)
    return chosen, cover, small


def _layer_fullsize(w: synth.Workload, tokens=None, n_tokens=16, max_experts=40,
                    cap_factor=0.0, layout="contiguous"):
    """``tokens``: the sampled tokens, or None to choose ``n_tokens`` of them spanning
    both GEMM tile classes with at most ``max_experts`` distinct experts."""
    note(f"full-size layer {w.name} T={w.T} d={w.d} E={w.E} k={w.k} I={w.I} "
         f"cap_factor={cap_factor} layout={layout}")
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
    elif w.mode == "w4a8":
        q13, s13 = M.moe_pack_weight_int4(q13, s13)
        q2, s2 = M.moe_pack_weight_int4(q2, s2)
    weights = {"w13": q13, "s13": s13, "w2": q2, "s2": s2}
    if w.route == "score":
        weights.update(w_router=inp["w_router"], bias=inp["bias"])
    desc = M.LayerDesc(w.T, w.d, w.E, w.k, w.I, mode=w.mode, route=w.route, m_align=w.m_align,
                       capacity_factor=cap_factor, layout=layout)
    y, counts = M.moe_layer_fwd(desc, weights, inp["x"], inp.get("token_ids"))
    staged = None
    if w.mode in ("fp8", "w4a8"):
        note(f"full-size layer {w.name}: the same steps through the individual entry points")
        staged = staged_fp8_layer(M, w.T, w.E, w.k, w.I, w.m_align, inp["x"], weights,
                                  capacity=M.moe_capacity(w.T, w.k, w.E, cap_factor),
                                  w4a8=w.mode == "w4a8", token_ids=inp.get("token_ids"))
        assert torch.equal(staged["y"], y) and torch.equal(staged["counts"], counts)
    torch.cuda.synchronize()
    del q13, q2
    ids = inp.get("token_ids")
    cnt = to_np(counts)
    near = np.zeros(w.T, bool)
    if w.route == "score":
        # routing of every token from the oracle's own fp64 logits (fp32-rounded)
        xs = inp["x"].float().cpu().numpy()
        logits = O.router_logits(xs, inp["w_router"].float().cpu().numpy()).astype(np.float32)
        key = (logits + inp["bias"].cpu().numpy()[None, :]).astype(np.float32).astype(np.float64)
        srt = -np.sort(-key, axis=1)
        near = (srt[:, w.k - 1] - srt[:, w.k]) < 1e-4
        print(f"near-tie tokens {int(near.sum())} of {w.T}")
    if tokens is None:
        gidx = to_np(staged["idx"]) if staged is not None else None
        tokens, cover, small = _pick_tokens(gidx, cnt, near, 16 if w.T * w.k / w.E <= 16
                                            else 32, n_tokens, max_experts)
        print(f"sampled tokens {len(tokens)}, experts {len(cover)} "
              f"({len(cover & small)} in small-row tiles)")
        live = set(np.nonzero(cnt)[0].tolist())
        assert len(tokens) >= n_tokens
        assert (cover & small or not small) and (cover - small or not live - small)
    tokens = [t for t in tokens if not near[t]]
    e13, e2 = LazyExperts(inp["w13"], w.mode), LazyExperts(inp["w2"], w.mode)
    if staged is not None:
        used = np.unique(to_np(staged["idx"])[tokens])
        e13.prefetch(used)
        e2.prefetch(used)
    experts = (e13.view(0), e13.view(1), e2.view(0), e2.view(1))
    ref = O.layer_forward(w.mode, inp["x"].float().cpu().numpy(), E=w.E, k=w.k, I=w.I,
                          m_align=w.m_align,
                          w_router=None if ids is not None else inp["w_router"].float().cpu().numpy(),
                          bias=None if ids is not None else inp["bias"].cpu().numpy(),
                          token_ids=None if ids is None else ids.cpu().numpy(),
                          experts=experts, tokens=tokens, keep=(w.mode in ("fp8", "w4a8")),
                          cap_factor=cap_factor)
    if w.route == "score":
        free = ~near
        np.testing.assert_array_equal(to_np(staged["idx"])[free], ref["idx"][free])
        n_checked = check_counts_outside_ties(cnt, ref, inp["bias"].cpu().numpy(), w.k, 1e-4)
        print(f"routing checked for {int(free.sum())} tokens, counts for {n_checked} experts")
    else:
        np.testing.assert_array_equal(cnt, ref["counts"])
    yg = to_np(y[tokens]).astype(np.float64)
    if w.mode in ("fp8", "w4a8"):
        h_gpu = gpu_h_by_slot(staged, [t * w.k + j for t in tokens for j in range(w.k)])
        e = fp8_layer_errors(yg, ref, np.asarray(tokens), w.T, w.k, h_gpu)
        print(f"errors {e}")
        assert e["beyond_flip"] <= TOL
        assert e["beyond_noflip"] <= TOL
    else:
        yr = ref["y"][tokens]
        r = 0.5 * ulp_bf16(yr)
        for i, t in enumerate(tokens):
            r[i] += 0.5 * ulp_bf16(ref["o_by_slot"][t])
        beyond, raw = error_ratios(yg, yr, rounding=r)
        print(f"beyond={beyond:.3e} raw={raw:.3e}")
        assert beyond <= TOL


def test_fullsize_prefill_layer():
    _layer_fullsize(synth.scaled(synth.WORKLOADS["prefill_fp8"], m_align=16), n_tokens=32,
                    max_experts=40)


def test_fullsize_decode_layer():
    _layer_fullsize(synth.WORKLOADS["decode_fp8"], n_tokens=12, max_experts=80)


def test_fullsize_decode_layer_masked():
    """The decode layer in the fixed-capacity layout, C = ceil(128*8/256) * 2 = 8."""
    _layer_fullsize(synth.WORKLOADS["decode_fp8"], n_tokens=12, max_experts=80,
                    cap_factor=2.0, layout="masked")


def test_fullsize_hash_w4a16_layer():
    _layer_fullsize(synth.WORKLOADS["hash_w4a16"], [0, 1, 4096, 8191])


def test_fullsize_hash_w4a8_layer():
    """The hash-routed 4-bit layer's shape (T=8192, d=4096, E=64, I=2048) with the weights
    kept 4-bit on the FP8 matrix core and 1x128 e4m3 activations."""
    _layer_fullsize(synth.WORKLOADS["hash_w4a8"], [0, 1, 77, 4096, 5000, 8191])


@pytest.mark.parametrize("big", ["0", "1"])
def test_fullsize_grouped_gemm_fp8(big, monkeypatch):
    """16 groups, sizes ~ Zipf(1.1) summing to 8192, each padded to 128; N=4096, K=7168.
    With big = "1" the whole 256-row tiles of the largest groups (one round of 16 row
    tiles) go to the 256 x 256-tile kernel and the rest to the 128-row kernel."""
    monkeypatch.setenv("FP8GG_BIG_TILES", big)
    sizes = synth.zipf_group_sizes(8192, 16, 1.1, seed=0)
    N, K = 4096, 7168
    note(f"full-size grouped GEMM sizes={sizes.tolist()} N={N} K={K} big={big}")
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
