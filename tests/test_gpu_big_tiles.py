"""GPU parity of the 256 x 256 tile path of the FP8 GEMM against the CPU oracle.

Groups averaging at least 256 rows send their whole 256-row tiles, in whole rounds of the
grid, to a second kernel; the rest of each group (and any big tiles past the last whole
round) stays with the 128/32/16-row kernel.  The shapes here are chosen so that both
kernels get work: enough whole 256-row tiles to fill at least one round (N = 4096 plain
gives 16 column tiles, so one round is 16 row tiles; SwiGLU N = 4096 gives 32 column
tiles and 8 row tiles a round), with big tiles left over and ragged group tails.  Each
case runs with the 256-row kernel switched on (FP8GG_BIG_TILES=1) and off (=0), and both
results are held to the same bound.
"""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as M
import oracle as O
from oracle import codecs as OC
import synth
from gpu_util import TOL, check_swiglu_codes, dev, error_ratios, note, to_np

pytestmark = pytest.mark.gpu

# m_align 16: 4 + 1 + 2 + 10 + 1 = 18 whole 256-row tiles (a round of 16 and 2 more)
SIZES = [1100, 0, 256, 700, 40, 2600, 300, 17]


def _case(sizes, N, K, seed, swiglu, m_align=16):
    sizes = np.asarray(sizes)
    padded = -(-sizes // m_align) * m_align
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    R = int(offsets[-1])
    a = synth.normal((R, K), seed, "gemm_a")
    for g in range(len(sizes)):
        a[offsets[g] + sizes[g]:offsets[g + 1]] = 0
    b = synth.normal((len(sizes), 2 * N if swiglu else N, K), seed, "gemm_b", std=K ** -0.5)
    live = np.zeros(R, bool)
    for g in range(len(sizes)):
        live[offsets[g]:offsets[g] + sizes[g]] = True
    return a, b, offsets, R, live


def _both_paths(monkeypatch, fn):
    """fn() with the 256-row kernel on, then off."""
    monkeypatch.setenv("FP8GG_BIG_TILES", "1")
    on = fn()
    torch.cuda.synchronize()
    monkeypatch.setenv("FP8GG_BIG_TILES", "0")
    off = fn()
    torch.cuda.synchronize()
    monkeypatch.delenv("FP8GG_BIG_TILES", raising=False)
    return on, off


@pytest.mark.parametrize("K", [256, 768])
@pytest.mark.parametrize("swiglu", [False, True])
def test_big_tiles_grouped(K, swiglu, monkeypatch):
    N = 4096
    note(f"big tiles grouped K={K} swiglu={swiglu}")
    a, b, offsets, R, live = _case(SIZES, N, K, 61, swiglu)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, sb = M.moe_quant_weight_fp8(b.to(dev()))
    bf = M.moe_pack_weight_fp8(qb)
    off_d = torch.from_numpy(offsets).to(dev())
    on, off = _both_paths(monkeypatch, lambda: M.grouped_gemm_fp8(qa, sa, bf, sb, off_d, R, N,
                                                                  swiglu=swiglu))
    qao, sao = OC.quant_fp8_act(a.numpy())
    qbo, sbo = OC.quant_fp8_weight(b.numpy())
    ref = O.grouped_gemm_fp8(qao, sao, qbo, sbo, offsets)
    if not swiglu:
        for name, c in (("256-row", on), ("128-row", off)):
            beyond, raw = error_ratios(to_np(c)[live], ref[live])
            print(f"{name}: beyond={beyond:.3e} raw={raw:.3e}")
            assert beyond <= TOL, (name, beyond)
        print("bit-identical to the 128-row kernel:", bool(torch.equal(on, off)))
    else:
        A = OC.dequant_fp8_act(qao, sao)
        Bd = OC.dequant_fp8_weight(qbo, sbo)
        sab = O.grouped_gemm(np.abs(A), np.abs(Bd), offsets)
        for codes, sc in (on, off):
            check_swiglu_codes(to_np(codes)[live], to_np(sc)[live], ref[live], sab[live], N)


def test_big_tiles_row_gather(monkeypatch):
    """GEMM1's gathered activation rows (a_rows, a_row_div) through the 256-row kernel."""
    N, K, k, T = 4096, 256, 2, 3000
    note("big tiles gather")
    sizes = np.asarray(SIZES)
    padded = -(-sizes // 16) * 16
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    R = int(offsets[-1])
    rng = np.random.default_rng(62)
    a_rows = np.full(R, -1, np.int32)
    for g in range(len(sizes)):
        a_rows[offsets[g]:offsets[g] + sizes[g]] = rng.integers(0, T * k, sizes[g])
    x = synth.normal((T, K), 62, "x", dtype=torch.bfloat16)
    w = synth.normal((len(sizes), N, K), 62, "w13", std=K ** -0.5)
    qx, sx = M.moe_quant_fp8(x.to(dev()))
    qw, sw = M.moe_quant_weight_fp8(w.to(dev()))
    bf = M.moe_pack_weight_fp8(qw)
    off_d = torch.from_numpy(offsets).to(dev())
    ar_d = torch.from_numpy(a_rows).to(dev())
    on, off = _both_paths(monkeypatch, lambda: M.grouped_gemm_fp8(
        qx, sx, bf, sw, off_d, R, N, a_rows=ar_d, a_row_div=k))
    qxo, sxo = OC.quant_fp8_act(x.float().numpy())
    qwo, swo = OC.quant_fp8_weight(w.numpy())
    live = a_rows >= 0
    A = np.zeros((R, K), np.uint8)
    sA = np.ones((R, K // 128), np.float32)
    A[live] = qxo[a_rows[live] // k]
    sA[live] = sxo[a_rows[live] // k]
    ref = O.grouped_gemm_fp8(A, sA, qwo, swo, offsets)
    for c in (on, off):
        beyond, raw = error_ratios(to_np(c)[live], ref[live])
        assert beyond <= TOL, beyond


@pytest.mark.parametrize("swiglu", [False, True])
def test_big_tiles_masked(swiglu, monkeypatch):
    """Fixed-capacity layout, cap 1280: 5 + 2 + 0 + 5 + 1 + 4 = 17 whole tiles (plain and
    SwiGLU N = 2048 both run 16 row tiles a round)."""
    G, cap, K = 6, 1280, 256
    N = 2048 if swiglu else 4096
    counts = np.array([1280, 600, 0, 1500, 300, 1100], np.int32)   # 1500 > cap: clamped
    note(f"big tiles masked swiglu={swiglu}")
    a = synth.normal((G * cap, K), 63, "gemm_a")
    b = synth.normal((G, 2 * N if swiglu else N, K), 63, "gemm_b", std=K ** -0.5)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, sb = M.moe_quant_weight_fp8(b.to(dev()))
    bf = M.moe_pack_weight_fp8(qb)
    cnt_d = torch.from_numpy(counts).to(dev())
    on, off = _both_paths(monkeypatch, lambda: M.grouped_gemm_fp8_masked(
        qa, sa, bf, sb, cnt_d, cap, N, swiglu=swiglu))
    qao, sao = OC.quant_fp8_act(a.numpy())
    qbo, sbo = OC.quant_fp8_weight(b.numpy())
    A = OC.dequant_fp8_act(qao, sao)
    Bd = OC.dequant_fp8_weight(qbo, sbo)
    for g in range(G):
        n = int(min(counts[g], cap))
        if n == 0:
            continue
        rows = slice(g * cap, g * cap + n)
        one = np.array([0, n], np.int32)
        ref = O.grouped_gemm_fp8(qao[rows], sao[rows], qbo[g:g + 1], sbo[g:g + 1], one)
        for out in (on, off):
            if not swiglu:
                beyond, raw = error_ratios(to_np(out)[rows], ref)
                assert beyond <= TOL, (g, beyond)
            else:
                sab = O.grouped_gemm(np.abs(A[rows]), np.abs(Bd[g:g + 1]), one)
                check_swiglu_codes(to_np(out[0])[rows], to_np(out[1])[rows], ref, sab, N)


@pytest.mark.parametrize("Mrows", [300, 4096, 4396])
def test_big_tiles_dense(Mrows, monkeypatch):
    """Dense GEMM: 300 rows (no whole round: the 256-row kernel finds nothing to do), 4096
    (one round, nothing left for the other kernel), 4396 (a round, a tile and a tail)."""
    N, K = 4096, 512
    note(f"big tiles dense M={Mrows}")
    a = synth.normal((Mrows, K), 64, "gemm_a")
    b = synth.normal((N, K), 64, "gemm_b", std=K ** -0.5)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, sb = M.moe_quant_weight_fp8(b[None].to(dev()))
    bf = M.moe_pack_weight_fp8(qb[0])
    on, off = _both_paths(monkeypatch, lambda: M.gemm_fp8(qa, sa, bf, sb[0]))
    qao, sao = OC.quant_fp8_act(a.numpy())
    qbo, sbo = OC.quant_fp8_weight(b[None].numpy())
    ref = O.grouped_gemm_fp8(qao, sao, qbo, sbo, np.array([0, Mrows], np.int32))
    for c in (on, off):
        beyond, raw = error_ratios(to_np(c), ref)
        print(f"beyond={beyond:.3e} raw={raw:.3e}")
        assert beyond <= TOL


def test_big_tiles_deterministic(monkeypatch):
    """Repeated calls give bit-identical output (fixed tile order, no atomics)."""
    monkeypatch.setenv("FP8GG_BIG_TILES", "1")
    N, K = 4096, 256
    note("big tiles determinism")
    a, b, offsets, R, live = _case(SIZES, N, K, 65, True)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, sb = M.moe_quant_weight_fp8(b.to(dev()))
    bf = M.moe_pack_weight_fp8(qb)
    off_d = torch.from_numpy(offsets).to(dev())
    c1, s1 = M.grouped_gemm_fp8(qa, sa, bf, sb, off_d, R, N, swiglu=True)
    c2, s2 = M.grouped_gemm_fp8(qa, sa, bf, sb, off_d, R, N, swiglu=True)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
