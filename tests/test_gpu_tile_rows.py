"""The FP8 GEMM's two large-tile sizes.  Groups above the small-tile size run in 192-row
tiles by default (128-row tiles for a dense M that they tile better, for K > 8192 and in
the 256-row mode); FP8GG_TILE_ROWS forces either size.  Both compute every output with
the same per-block MFMA, promotion order and epilogue arithmetic, so they must agree bit
for bit; the default path is checked against the oracle by the other GEMM and layer
tests, and the 128-row path against the oracle here as well."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as M
import oracle as O
from oracle import codecs as OC
import synth
from gpu_util import TOL, dev, error_ratios, note, to_np

pytestmark = pytest.mark.gpu


def _case(sizes, N, K, m_align, seed, swiglu):
    sizes = np.asarray(sizes)
    padded = -(-sizes // m_align) * m_align
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    R = int(offsets[-1])
    a = synth.normal((max(R, 1), K), seed, "gemm_a")
    b = synth.normal((len(sizes), 2 * N if swiglu else N, K), seed, "gemm_b", std=K ** -0.5)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, sb = M.moe_quant_weight_fp8(b.to(dev()))
    return a, b, qa, sa, qb, sb, offsets, R


def _both(monkeypatch, fn, rows=None, heights=("128", "192")):
    """fn() under each FP8GG_TILE_ROWS value in ``heights`` and unset: equal bit for bit
    (on the output rows a call writes: all, or the boolean mask ``rows``)."""
    out = {}
    for tr in heights:
        monkeypatch.setenv("FP8GG_TILE_ROWS", tr)
        r = fn()
        torch.cuda.synchronize()
        out[tr] = [t.clone() for t in (r if isinstance(r, tuple) else (r,))]
    monkeypatch.delenv("FP8GG_TILE_ROWS")
    d = fn()
    torch.cuda.synchronize()
    out["default"] = [t.clone() for t in (d if isinstance(d, tuple) else (d,))]
    keep = torch.from_numpy(rows).to(dev()) if rows is not None else None
    for tr in list(heights[1:]) + ["default"]:
        for x, y in zip(out[heights[0]], out[tr]):
            if keep is not None:
                x, y = x[keep], y[keep]
            assert torch.equal(x, y), tr
    return out[heights[0]]


@pytest.mark.parametrize("sizes,m_align,K", [
    ([128, 256, 64, 512, 128, 256, 64, 512], 128, 512),
    ([0, 1, 17, 130, 300, 0, 193, 385, 191], 16, 1024),   # empty, tiny, ragged, 192 +/- 1
    ([700, 20, 1100, 5, 384], 16, 7168),                    # prefill-like mix, K = d
    ([900, 33, 600], 16, 2048),                             # K = I
    ([400, 250], 16, 8192),                                 # the 192-row tiles' largest K
    ([400, 250], 16, 8320),                                 # past it: 128-row tiles only
    ([200, 64, 1], 16, 128),                                # a single K block
])
@pytest.mark.parametrize("swiglu", [False, True])
def test_tile_rows_bit_identical(sizes, m_align, K, swiglu, monkeypatch):
    N = 256
    note(f"tile rows sizes={sizes} K={K} swiglu={swiglu}")
    a, b, qa, sa, qb, sb, offsets, R = _case(sizes, N, K, m_align, 21, swiglu)
    off_d = torch.from_numpy(offsets).to(dev())
    qbp = M.moe_pack_weight_fp8(qb)
    _both(monkeypatch, lambda: M.grouped_gemm_fp8(qa, sa, qbp, sb, off_d, R, N, swiglu=swiglu))


def test_tile_rows_128_against_oracle(monkeypatch):
    """The 128-row path, forced, against the oracle (plain output)."""
    sizes, N, K = [300, 17, 129, 640], 256, 1024
    note("tile rows 128 vs oracle")
    a, b, qa, sa, qb, sb, offsets, R = _case(sizes, N, K, 16, 22, False)
    monkeypatch.setenv("FP8GG_TILE_ROWS", "128")
    c = M.grouped_gemm_fp8(qa, sa, M.moe_pack_weight_fp8(qb), sb,
                           torch.from_numpy(offsets).to(dev()), R, N)
    torch.cuda.synchronize()
    qao, sao = OC.quant_fp8_act(a.numpy())
    qbo, sbo = OC.quant_fp8_weight(b.numpy())
    ref = O.grouped_gemm_fp8(qao, sao, qbo, sbo, offsets)
    live = np.zeros(R, bool)
    for g in range(len(sizes)):
        live[offsets[g]:offsets[g] + sizes[g]] = True
    beyond, raw = error_ratios(to_np(c)[live], ref[live])
    print(f"beyond={beyond:.3e} raw={raw:.3e}")
    assert beyond <= TOL


@pytest.mark.parametrize("swiglu", [False, True])
def test_tile_rows_masked_and_gather(swiglu, monkeypatch):
    """Fixed-capacity layout and the row gather (GEMM1's activation read through the
    dispatch map) in both tile sizes."""
    note(f"tile rows masked/gather swiglu={swiglu}")
    N, K, cap = 128, 1024, 400
    counts = torch.tensor([400, 0, 193, 37, 250], dtype=torch.int32, device=dev())
    G = counts.numel()
    a = synth.normal((G * cap, K), 23, "gemm_a")
    b = synth.normal((G, 2 * N if swiglu else N, K), 23, "gemm_b", std=K ** -0.5)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, sb = M.moe_quant_weight_fp8(b.to(dev()))
    qbp = M.moe_pack_weight_fp8(qb)
    written = np.zeros(G * cap, bool)               # rows past a group's count are not
    for g, c in enumerate(counts.tolist()):          # written by the masked GEMM
        written[g * cap:g * cap + c] = True
    _both(monkeypatch,
          lambda: M.grouped_gemm_fp8_masked(qa, sa, qbp, sb, counts, cap, N, swiglu=swiglu),
          rows=written)
    T, k, E = 600, 2, 4
    idx = synth.random_topk(T, E, k, seed=5, skew=1.1)
    cnt, offsets, ros, sor = O.dispatch(idx, E, 16)
    x = synth.normal((T, K), 23, "x", dtype=torch.bfloat16)
    w = synth.normal((E, 2 * N if swiglu else N, K), 23, "w13", std=K ** -0.5)
    qx, sx = M.moe_quant_fp8(x.to(dev()))
    qw, sw = M.moe_quant_weight_fp8(w.to(dev()))
    qwp = M.moe_pack_weight_fp8(qw)
    off_d = torch.from_numpy(offsets).to(dev())
    sor_d = torch.from_numpy(sor).to(dev())
    print(f"gather counts {cnt.tolist()}")
    # (rows past the last group's padded end belong to no group and are not written)
    _both(monkeypatch,
          lambda: M.grouped_gemm_fp8(qx, sx, qwp, sw, off_d, len(sor), N, swiglu=swiglu,
                                     a_rows=sor_d, a_row_div=k),
          rows=np.arange(len(sor)) < offsets[-1])


@pytest.mark.parametrize("Mrows", [8192, 8256, 1000, 193])
def test_tile_rows_dense(Mrows, monkeypatch):
    note(f"tile rows dense M={Mrows}")
    N, K = 512, 1024
    a = synth.normal((Mrows, K), 24, "gemm_a")
    b = synth.normal((1, N, K), 24, "gemm_b", std=K ** -0.5)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, sb = M.moe_quant_weight_fp8(b.to(dev()))
    qbp = M.moe_pack_weight_fp8(qb)
    _both(monkeypatch, lambda: M.gemm_fp8(qa, sa, qbp[0], sb[0]))


@pytest.mark.parametrize("swiglu", [False, True])
def test_tile_rows_w4a8(swiglu, monkeypatch):
    """The 4-bit-weight instance in its three tile heights (hash-layer-like groups of ~128
    rows, one of 193)."""
    note(f"tile rows w4a8 swiglu={swiglu}")
    sizes, N, K = [120, 150, 0, 131, 193, 17], 256, 2048
    a, b, qa, sa, _, _, offsets, R = _case(sizes, N, K, 16, 25, swiglu)
    qf, s7f = M.moe_pack_weight_int4(*M.moe_quant_weight_int4(b.to(dev())))
    off_d = torch.from_numpy(offsets).to(dev())
    _both(monkeypatch,
          lambda: M.grouped_gemm_w4a8(qa, sa, qf, s7f, off_d, R, N, swiglu=swiglu),
          heights=("128", "160", "192"))
