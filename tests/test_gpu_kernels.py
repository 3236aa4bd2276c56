"""GPU parity of every C-ABI step against the CPU oracle on the same seeded inputs.

Integer results (codes, indices, counts, offsets, permutations) must be bit-exact;
floating-point results are held to max|err beyond the prescribed output rounding| /
max|ref| <= 2e-3 (the raw ratio is reported beside it).
"""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as M
import oracle as O
from oracle import codecs as OC
import synth
from gpu_util import (TOL, check_swiglu_codes, dev, error_ratios, note, requant_band,
                      swiglu_error_model, to_np)

pytestmark = pytest.mark.gpu


# -------------------------------------------------------------- quantisation

def test_e4m3_conversion_every_boundary():
    """Blocks whose largest element is 448 have scale 1, so the codes are the direct
    conversion of the other 127 values: sweep every representable value, every
    midpoint (ties) and its neighbours one fp32 ulp away."""
    note("e4m3 conversion sweep")
    t = OC.e4m3_decode_table()
    pos = np.sort(np.unique(np.abs(t[np.isfinite(t)])))
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([pos, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9)),
                           np.float32([1e-30, 2.0 ** -12, 3 * 2.0 ** -11, 447.9, 440.0])])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    n = len(vals)
    nblk = (n + 126) // 127
    x = np.zeros((nblk, 128), np.float32)
    flat = np.zeros(nblk * 127, np.float32)
    flat[:n] = vals
    x[:, 1:] = flat.reshape(nblk, 127)
    x[:, 0] = 448.0
    q, s = M.moe_quant_fp8(torch.from_numpy(x).to(dev()))
    qo, so = OC.quant_fp8_act(x)
    np.testing.assert_array_equal(to_np(s), so)
    assert np.all(so == 1.0)
    np.testing.assert_array_equal(to_np(q), qo)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quant_act_bitexact(dtype):
    note(f"quant act {dtype}")
    x = synth.normal((37, 640), 5, "x", dtype=dtype)
    x[3, 128:256] = 0                        # all-zero block -> scale 1, zero codes
    x[4, :128] *= 1e-3
    x[5, 256:384] *= 300.0
    q, s = M.moe_quant_fp8(x.to(dev()))
    qo, so = OC.quant_fp8_act(x.float().numpy())
    np.testing.assert_array_equal(to_np(s), so)
    np.testing.assert_array_equal(to_np(q), qo)


def test_quant_act_gather():
    note("quant act gather")
    T, k, K = 21, 3, 256
    x = synth.normal((T, K), 6, "x", dtype=torch.bfloat16)
    src = np.array([5, -1, 62, 0, 11, -1, 30, 45], np.int32)   # slots; token = slot // k
    q, s = M.moe_quant_fp8(x.to(dev()), torch.from_numpy(src).to(dev()), k, len(src))
    qo, so = OC.quant_fp8_act(x.float().numpy())
    for r, sl in enumerate(src):
        if sl < 0:
            assert np.all(to_np(q[r]) == 0) and np.all(to_np(s[r]) == 1.0)
        else:
            np.testing.assert_array_equal(to_np(q[r]), qo[sl // k])
            np.testing.assert_array_equal(to_np(s[r]), so[sl // k])


def test_quant_weight_fp8_bitexact():
    note("quant weight fp8")
    w = synth.normal((3, 256, 384), 7, "w13", std=0.02)
    w[1, :128, :128] = 0
    q, s = M.moe_quant_weight_fp8(w.to(dev()))
    qo, so = OC.quant_fp8_weight(w.numpy())
    np.testing.assert_array_equal(to_np(s), so)
    np.testing.assert_array_equal(to_np(q), qo)


def _pack_reference(q):
    """The fragment-major layout written out with numpy: [G][N/16][K/128][2][64][16]
    with half h, lane l of block (nb, kb) holding row 16 nb + l % 16, columns
    128 kb + 32 (l // 16) + 16 h .. +16."""
    G, N, K = q.shape
    x = q.reshape(G, N // 16, 16, K // 128, 4, 2, 16)      # g, nb, r, kb, c, h, byte
    x = x.transpose(0, 1, 3, 5, 4, 2, 6)                   # g, nb, kb, h, c, r, byte
    return np.ascontiguousarray(x).reshape(G, N, K)        # lane = 16 c + r


@pytest.mark.parametrize("shape", [(1, 128, 128), (3, 256, 384), (2, 384, 1024)])
def test_pack_weight_fp8_permutation(shape):
    note(f"pack weight fp8 {shape}")
    q = torch.randint(0, 256, shape, dtype=torch.uint8, generator=torch.Generator().manual_seed(5))
    qf = M.moe_pack_weight_fp8(q.to(dev()))
    np.testing.assert_array_equal(to_np(qf), _pack_reference(q.numpy()))
    # a [N, K] matrix packs as one group
    q2 = M.moe_pack_weight_fp8(q[0].to(dev()))
    np.testing.assert_array_equal(to_np(q2), _pack_reference(q[:1].numpy())[0])


def test_quant_weight_int4_bitexact():
    note("quant weight int4")
    w = synth.normal((2, 40, 384), 8, "w2", std=0.02)
    w[0, 3, :128] = 0
    q, s7 = M.moe_quant_weight_int4(w.to(dev()))
    qo, so = OC.int4_quant_rows(w.numpy())
    np.testing.assert_array_equal(to_np(s7), so)
    np.testing.assert_array_equal(to_np(q), OC.int4_pack(qo))


# -------------------------------------------------------------------- routing

@pytest.mark.parametrize("T,E,k,ties,renorm", [(300, 256, 8, False, False),
                                               (300, 256, 8, True, False),
                                               (77, 8, 2, True, True),
                                               (50, 64, 6, False, True),
                                               (40, 1000, 7, True, False),
                                               (33, 5, 5, False, False)])
def test_route_from_logits(T, E, k, ties, renorm):
    note(f"topk T={T} E={E} k={k} ties={ties} renorm={renorm}")
    L = synth.random_logits(T, E, seed=E + k, ties=ties)
    b = synth.uniform((E,), -0.01, 0.01, 3, "bias")
    if ties:
        b = torch.round(b * 100) / 100 * 0   # keep exact ties in the keys
    idx, w = M.moe_route_from_logits(L.to(dev()), b.to(dev()), k, renorm)
    io, wo = O.topk_route(L.numpy(), b.numpy(), k, renorm)
    np.testing.assert_array_equal(to_np(idx), io)
    # fp32 softmax vs fp64: a few ulp per exp and per partial sum
    np.testing.assert_allclose(to_np(w), wo, rtol=2e-5, atol=0)


@pytest.mark.parametrize("dtype,T,d,E,k,ws", [(torch.bfloat16, 200, 512, 256, 8, True),
                                              (torch.bfloat16, 70, 7168, 64, 6, True),
                                              (torch.bfloat16, 128, 7168, 256, 8, True),
                                              (torch.bfloat16, 300, 7168, 256, 8, True),
                                              (torch.bfloat16, 4096, 7168, 256, 8, True),
                                              (torch.bfloat16, 1, 128, 300, 4, True),
                                              (torch.bfloat16, 129, 1024, 520, 8, True),
                                              (torch.bfloat16, 257, 2048, 256, 8, False),
                                              (torch.float32, 256, 256, 8, 2, True)])
def test_router_logits(dtype, T, d, E, k, ws):
    """Logits within the fp32 accumulation bound; routing equal to the oracle's own
    routing wherever the k-th and (k+1)-th keys are further apart than that bound (and
    a valid choice where they are not).  Covers the split-K partial logits, partial
    token and expert tiles, and the unsplit GEMM when no workspace is given."""
    note(f"router logits {dtype} T={T} d={d} E={E} k={k} ws={ws}")
    x = synth.normal((T, d), 9, "x", dtype=dtype)
    w = synth.normal((E, d), 9, "w_gate_router", std=d ** -0.5, dtype=dtype)
    b = synth.uniform((E,), -0.01, 0.01, 9, "bias")
    idx, gw, logits = M.moe_route(x.to(dev()), w.to(dev()), b.to(dev()), k, use_workspace=ws)
    ref = O.router_logits(x.float().numpy(), w.float().numpy())
    # fp32 accumulation of d exact products: |err| <= d * 2^-24 * sum|x_i w_i|
    bound = d * 2.0 ** -24 * (np.abs(x.float().numpy()) @ np.abs(w.float().numpy()).T)
    assert np.all(np.abs(to_np(logits) - ref) <= bound + 1e-30)
    L32 = ref.astype(np.float32)
    io, wo = O.topk_route(L32, b.numpy(), k)
    key = (L32 + b.numpy()[None, :]).astype(np.float64)
    srt = -np.sort(-key, axis=1)
    margin = 2 * bound.max(axis=1) + 4 * np.abs(srt[:, 0]) * 2.0 ** -24
    clear = (srt[:, k - 1] - srt[:, k]) > margin
    gi = to_np(idx)
    np.testing.assert_array_equal(gi[clear], io[clear])
    for t in np.nonzero(~clear)[0]:          # near ties: any choice within the margin
        assert np.all(key[t, gi[t]] >= srt[t, k - 1] - margin[t])
    print(f"tokens with a near tie: {int((~clear).sum())}")
    np.testing.assert_allclose(to_np(gw)[clear], wo[clear], rtol=1e-4)


def test_hash_route():
    note("hash route")
    ids = torch.randint(0, 129280, (5000,), generator=torch.Generator().manual_seed(1),
                        dtype=torch.int64)
    ids[:4] = torch.tensor([0, 1, 2, 2 ** 40 + 7])
    idx, w = M.moe_route_hash(ids.to(dev()), 64)
    io, wo = O.hash_route(ids.numpy(), 64)
    np.testing.assert_array_equal(to_np(idx), io)
    assert np.all(to_np(w) == 1.0)


# ------------------------------------------------------------------- dispatch

@pytest.mark.parametrize("T,E,k,m_align,cap", [(4096, 256, 8, 128, 0), (128, 256, 8, 16, 0),
                                               (500, 64, 1, 128, 0), (333, 13, 3, 32, 0),
                                               (333, 13, 3, 16, 40), (1, 4, 2, 1, 0),
                                               (0, 4, 2, 16, 0), (2048, 64, 2, 64, 76),
                                               (300, 400, 4, 16, 0), (200, 700, 2, 16, 9),
                                               (16384, 256, 8, 16, 300)])
def test_dispatch_bitexact(T, E, k, m_align, cap):
    note(f"dispatch T={T} E={E} k={k} m_align={m_align} cap={cap}")
    idx = synth.random_topk(T, E, k, seed=T + E, skew=1.1) if T else np.zeros((0, k), np.int32)
    counts, offsets, ros, sor = M.moe_dispatch(torch.from_numpy(idx).to(dev()), E, m_align, cap)
    co, oo, ro, so = O.dispatch(idx, E, m_align, cap)
    np.testing.assert_array_equal(to_np(counts), co)
    np.testing.assert_array_equal(to_np(offsets), oo)
    np.testing.assert_array_equal(to_np(ros), ro)
    np.testing.assert_array_equal(to_np(sor), so)


@pytest.mark.parametrize("T,E,k,cap", [(128, 256, 8, 8), (333, 13, 3, 40), (333, 13, 3, 200),
                                       (200, 700, 2, 3), (1, 4, 2, 1), (4096, 256, 8, 160)])
def test_dispatch_masked_bitexact(T, E, k, cap):
    """Fixed-capacity layout: counts, row_of_slot and slot_of_row [E*C] bit-exact, with and
    without drops, on the one-workgroup kernel and the per-expert kernels (E > 512)."""
    note(f"dispatch masked T={T} E={E} k={k} cap={cap}")
    idx = synth.random_topk(T, E, k, seed=T + E + 1, skew=1.1)
    counts, ros, sor = M.moe_dispatch_masked(torch.from_numpy(idx).to(dev()), E, cap)
    co, ro, so = O.dispatch_masked(idx, E, cap)
    np.testing.assert_array_equal(to_np(counts), co)
    np.testing.assert_array_equal(to_np(ros), ro)
    np.testing.assert_array_equal(to_np(sor), so)


# ---------------------------------------------------------------- grouped GEMM

def _gemm_case(sizes, N, K, m_align, seed, swiglu):
    sizes = np.asarray(sizes)
    G = len(sizes)
    padded = -(-sizes // m_align) * m_align
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    R = int(offsets[-1]) + 7                      # a few rows past the last group
    a = synth.normal((R, K), seed, "gemm_a")
    for g in range(G):                            # padding rows hold zeros
        a[offsets[g] + sizes[g]:offsets[g + 1]] = 0
    Nb = 2 * N if swiglu else N
    b = synth.normal((G, Nb, K), seed, "gemm_b", std=K ** -0.5)
    return a, b, offsets, R


@pytest.mark.parametrize("sizes,m_align", [
    ([128, 256, 64, 512, 128, 256, 64, 512], 128),   # the page's group-size example
    ([0, 1, 17, 130, 300, 0], 16),                     # empty, tiny, ragged groups
    ([5, 3, 9, 2, 7, 1, 4, 6, 8, 3], 8),              # decode-sized groups (bm 16)
    ([40, 33, 50, 20], 32),                            # bm 32
    ([90, 70, 100], 64),                               # bm 64
])
@pytest.mark.parametrize("swiglu", [False, True])
def test_grouped_gemm_fp8(sizes, m_align, swiglu):
    N, K = 256, 512
    note(f"gemm fp8 sizes={sizes} m_align={m_align} swiglu={swiglu}")
    a, b, offsets, R = _gemm_case(sizes, N, K, m_align, 11, swiglu)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, sb = M.moe_quant_weight_fp8(b.to(dev()))
    qao, sao = OC.quant_fp8_act(a.numpy())
    qbo, sbo = OC.quant_fp8_weight(b.numpy())
    np.testing.assert_array_equal(to_np(qa), qao)
    np.testing.assert_array_equal(to_np(qb), qbo)
    off_d = torch.from_numpy(offsets).to(dev())
    ref = O.grouped_gemm_fp8(qao, sao, qbo, sbo, offsets)
    live = np.zeros(R, bool)
    for g in range(len(sizes)):
        live[offsets[g]:offsets[g] + sizes[g]] = True
    if not swiglu:
        c = M.grouped_gemm_fp8(qa, sa, M.moe_pack_weight_fp8(qb), sb, off_d, R, N)
        beyond, raw = error_ratios(to_np(c)[live], ref[live])
        print(f"beyond={beyond:.3e} raw={raw:.3e}")
        assert beyond <= TOL
    else:
        codes, sc = M.grouped_gemm_fp8(qa, sa, M.moe_pack_weight_fp8(qb), sb, off_d, R, N,
                                       swiglu=True)
        A = OC.dequant_fp8_act(qao, sao)
        Bd = OC.dequant_fp8_weight(qbo, sbo)
        sab = O.grouped_gemm(np.abs(A), np.abs(Bd), offsets)      # sum_k |a_k b_k|
        h, dh = swiglu_error_model(ref[:, :N], ref[:, N:], sab[:, :N], sab[:, N:])
        q, s, q_lo, q_hi, delta, rho = requant_band(h[live], dh[live])
        qg, sg = to_np(codes)[live], to_np(sc)[live]
        # the GPU scale is fl32(amax/448) of its own h: within the amax error band
        assert np.all(np.abs(sg.astype(np.float64) - s) <= s * rho * 1.01)
        dg = OC.e4m3_decode(qg)
        ok = (dg >= np.minimum(OC.e4m3_decode(q_lo), OC.e4m3_decode(q_hi))) & \
             (dg <= np.maximum(OC.e4m3_decode(q_lo), OC.e4m3_decode(q_hi)))
        unique = q_lo == q_hi
        print(f"unambiguous codes {unique.mean():.6f}, all codes valid {ok.mean():.6f}")
        # where the rounding is unambiguous the code is bit-exact; elsewhere it is one
        # of the correct neighbours
        np.testing.assert_array_equal(qg[unique], q[unique])
        assert ok.all()


def test_grouped_gemm_fp8_row_gather():
    """GEMM1's activation gather: logical row r reads A row a_rows[r] // div."""
    note("gemm fp8 gather")
    T, k, E, N, K = 50, 2, 4, 128, 256
    idx = synth.random_topk(T, E, k, seed=4)
    counts, offsets, ros, sor = O.dispatch(idx, E, 16)
    x = synth.normal((T, K), 12, "x", dtype=torch.bfloat16)
    w = synth.normal((E, N, K), 12, "w13", std=K ** -0.5)
    qx, sx = M.moe_quant_fp8(x.to(dev()))
    qw, sw = M.moe_quant_weight_fp8(w.to(dev()))
    R = len(sor)
    c = M.grouped_gemm_fp8(qx, sx, M.moe_pack_weight_fp8(qw), sw,
                           torch.from_numpy(offsets).to(dev()), R, N,
                           a_rows=torch.from_numpy(sor).to(dev()), a_row_div=k)
    qxo, sxo = OC.quant_fp8_act(x.float().numpy())
    qwo, swo = OC.quant_fp8_weight(w.numpy())
    live = sor >= 0
    A = np.zeros((R, K), np.uint8)
    sA = np.ones((R, K // 128), np.float32)
    A[live] = qxo[sor[live] // k]
    sA[live] = sxo[sor[live] // k]
    ref = O.grouped_gemm_fp8(A, sA, qwo, swo, offsets)
    beyond, raw = error_ratios(to_np(c)[live], ref[live])
    assert beyond <= TOL


@pytest.mark.parametrize("swiglu", [False, True])
def test_grouped_gemm_fp8_masked(swiglu):
    """Fixed-capacity layout: group g owns rows [g*cap, g*cap + min(counts[g], cap))."""
    G, cap, N, K = 5, 48, 128, 384
    counts = np.array([0, 1, 48, 60, 17], np.int32)          # 60 > cap: clamped
    note(f"gemm fp8 masked swiglu={swiglu}")
    a = synth.normal((G * cap, K), 21, "gemm_a")
    Nb = 2 * N if swiglu else N
    b = synth.normal((G, Nb, K), 21, "gemm_b", std=K ** -0.5)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, sb = M.moe_quant_weight_fp8(b.to(dev()))
    qao, sao = OC.quant_fp8_act(a.numpy())
    qbo, sbo = OC.quant_fp8_weight(b.numpy())
    out = M.grouped_gemm_fp8_masked(qa, sa, M.moe_pack_weight_fp8(qb), sb,
                                    torch.from_numpy(counts).to(dev()), cap, N, swiglu=swiglu)
    A = OC.dequant_fp8_act(qao, sao)
    Bd = OC.dequant_fp8_weight(qbo, sbo)
    for g in range(G):
        n = int(min(counts[g], cap))
        if n == 0:
            continue
        rows = slice(g * cap, g * cap + n)
        one = np.array([0, n], np.int32)
        ref = O.grouped_gemm_fp8(qao[rows], sao[rows], qbo[g:g + 1], sbo[g:g + 1], one)
        if not swiglu:
            beyond, raw = error_ratios(to_np(out)[rows], ref)
            assert beyond <= TOL, (g, beyond)
        else:
            sab = O.grouped_gemm(np.abs(A[rows]), np.abs(Bd[g:g + 1]), one)
            check_swiglu_codes(to_np(out[0])[rows], to_np(out[1])[rows], ref, sab, N)


@pytest.mark.parametrize("K", [128, 256, 384, 640, 1536])
@pytest.mark.parametrize("sizes,m_align", [
    ([3, 20, 40, 150], 16),        # 32-row tiles (six-block weight ring) and 128-row tiles
    ([1, 5, 9, 16, 2], 8),         # 16-row tiles
])
@pytest.mark.parametrize("swiglu", [False, True])
def test_grouped_gemm_fp8_short_k(K, sizes, m_align, swiglu):
    """K with fewer 128-deep blocks than the weight ring and the unrolled K loop: every
    block count from 1 up, tails of every length."""
    N = 128 if swiglu else 256
    note(f"gemm fp8 short K={K} sizes={sizes} swiglu={swiglu}")
    a, b, offsets, R = _gemm_case(sizes, N, K, m_align, 31, swiglu)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, sb = M.moe_quant_weight_fp8(b.to(dev()))
    qao, sao = OC.quant_fp8_act(a.numpy())
    qbo, sbo = OC.quant_fp8_weight(b.numpy())
    off_d = torch.from_numpy(offsets).to(dev())
    ref = O.grouped_gemm_fp8(qao, sao, qbo, sbo, offsets)
    live = np.zeros(R, bool)
    for g in range(len(sizes)):
        live[offsets[g]:offsets[g] + sizes[g]] = True
    if not swiglu:
        c = M.grouped_gemm_fp8(qa, sa, M.moe_pack_weight_fp8(qb), sb, off_d, R, N)
        beyond, raw = error_ratios(to_np(c)[live], ref[live])
        assert beyond <= TOL, beyond
    else:
        codes, sc = M.grouped_gemm_fp8(qa, sa, M.moe_pack_weight_fp8(qb), sb, off_d, R, N,
                                       swiglu=True)
        A = OC.dequant_fp8_act(qao, sao)
        Bd = OC.dequant_fp8_weight(qbo, sbo)
        sab = O.grouped_gemm(np.abs(A), np.abs(Bd), offsets)
        check_swiglu_codes(to_np(codes)[live], to_np(sc)[live], ref[live], sab[live], N)


@pytest.mark.parametrize("case", ["max_k", "max_groups"])
def test_grouped_gemm_fp8_limits(case):
    """The largest K the kernel accepts (16384: the tile's activation-scale table full)
    and the largest group count (1024, mixed small and large groups, so both tile lists
    and their interleave span the whole tile map)."""
    if case == "max_k":
        sizes, N, K, m_align = [3, 0, 150, 20], 128, 16384, 16
    else:
        rng = np.random.default_rng(12)
        sizes = rng.integers(0, 24, 1024)
        sizes[rng.choice(1024, 12, replace=False)] = rng.integers(100, 300, 12)
        sizes = sizes.tolist()
        N, K, m_align = 128, 256, 16
    for swiglu in (False, True):
        note(f"gemm fp8 limits {case} swiglu={swiglu}")
        a, b, offsets, R = _gemm_case(sizes, N, K, m_align, 41, swiglu)
        qa, sa = M.moe_quant_fp8(a.to(dev()))
        qb, sb = M.moe_quant_weight_fp8(b.to(dev()))
        qao, sao = OC.quant_fp8_act(a.numpy())
        qbo, sbo = OC.quant_fp8_weight(b.numpy())
        off_d = torch.from_numpy(offsets).to(dev())
        ref = O.grouped_gemm_fp8(qao, sao, qbo, sbo, offsets)
        live = np.zeros(R, bool)
        for g in range(len(sizes)):
            live[offsets[g]:offsets[g] + sizes[g]] = True
        if not swiglu:
            c = M.grouped_gemm_fp8(qa, sa, M.moe_pack_weight_fp8(qb), sb, off_d, R, N)
            beyond, raw = error_ratios(to_np(c)[live], ref[live])
            assert beyond <= TOL, beyond
        else:
            codes, sc = M.grouped_gemm_fp8(qa, sa, M.moe_pack_weight_fp8(qb), sb, off_d, R, N,
                                           swiglu=True)
            A = OC.dequant_fp8_act(qao, sao)
            Bd = OC.dequant_fp8_weight(qbo, sbo)
            sab = O.grouped_gemm(np.abs(A), np.abs(Bd), offsets)
            check_swiglu_codes(to_np(codes)[live], to_np(sc)[live], ref[live], sab[live], N)


@pytest.mark.parametrize("K", [8192, 8320])
@pytest.mark.parametrize("swiglu", [False, True])
def test_grouped_gemm_fp8_scale_table_forms(K, swiglu):
    """Both sides of the K at which 128-row tiles stop keeping row-scale x weight-scale
    products in LDS (64 blocks) and form the products in the K loop: mixed 32- and
    128-row tiles; plain N = 384 ends on a half column tile (one weight-scale block)."""
    sizes, m_align = [150, 20, 260, 0, 7], 16
    N = 256 if swiglu else 384
    note(f"gemm fp8 table forms K={K} swiglu={swiglu}")
    a, b, offsets, R = _gemm_case(sizes, N, K, m_align, 53, swiglu)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, sb = M.moe_quant_weight_fp8(b.to(dev()))
    qao, sao = OC.quant_fp8_act(a.numpy())
    qbo, sbo = OC.quant_fp8_weight(b.numpy())
    off_d = torch.from_numpy(offsets).to(dev())
    ref = O.grouped_gemm_fp8(qao, sao, qbo, sbo, offsets)
    live = np.zeros(R, bool)
    for g in range(len(sizes)):
        live[offsets[g]:offsets[g] + sizes[g]] = True
    if not swiglu:
        c = M.grouped_gemm_fp8(qa, sa, M.moe_pack_weight_fp8(qb), sb, off_d, R, N)
        beyond, raw = error_ratios(to_np(c)[live], ref[live])
        assert beyond <= TOL, beyond
    else:
        codes, sc = M.grouped_gemm_fp8(qa, sa, M.moe_pack_weight_fp8(qb), sb, off_d, R, N,
                                       swiglu=True)
        A = OC.dequant_fp8_act(qao, sao)
        Bd = OC.dequant_fp8_weight(qbo, sbo)
        sab = O.grouped_gemm(np.abs(A), np.abs(Bd), offsets)
        check_swiglu_codes(to_np(codes)[live], to_np(sc)[live], ref[live], sab[live], N)


@pytest.mark.parametrize("Mrows,K", [(0, 512), (1, 512), (200, 512), (333, 512),
                                     (333, 128), (40, 256), (333, 640)])
def test_gemm_fp8_dense(Mrows, K):
    N = 384
    note(f"gemm fp8 dense M={Mrows} K={K}")
    a = synth.normal((max(Mrows, 1), K), 22, "gemm_a")[:Mrows]
    b = synth.normal((N, K), 22, "gemm_b", std=K ** -0.5)
    qa, sa = M.moe_quant_fp8(a.to(dev())) if Mrows else (
        torch.empty((0, K), dtype=torch.uint8, device=dev()),
        torch.empty((0, K // 128), dtype=torch.float32, device=dev()))
    qb, sb = M.moe_quant_weight_fp8(b[None].to(dev()))
    c = M.gemm_fp8(qa, sa, M.moe_pack_weight_fp8(qb[0]), sb[0])
    assert tuple(c.shape) == (Mrows, N)
    if Mrows == 0:
        return
    qao, sao = OC.quant_fp8_act(a.numpy())
    qbo, sbo = OC.quant_fp8_weight(b[None].numpy())
    ref = O.grouped_gemm_fp8(qao, sao, qbo, sbo, np.array([0, Mrows], np.int32))
    beyond, raw = error_ratios(to_np(c), ref)
    print(f"beyond={beyond:.3e} raw={raw:.3e}")
    assert beyond <= TOL


@pytest.mark.parametrize("K", [128, 256, 384, 512, 1280])
@pytest.mark.parametrize("swiglu", [False, True])
def test_grouped_gemm_w4a16(swiglu, K):
    """Every K-block count of the three-stage pipeline (1, 2, 3, 4 and 10 blocks) and all
    three tile variants (<= 32, <= 64 and 128 live rows)."""
    sizes = [70, 0, 130, 5, 40]
    N = 128
    note(f"gemm w4a16 swiglu={swiglu} K={K}")
    a, b, offsets, R = _gemm_case(sizes, N, K, 16, 13, swiglu)
    a_bf = a.to(torch.bfloat16)
    qb, s7 = M.moe_quant_weight_int4(b.to(dev()))
    qbo, s7o = OC.int4_quant_rows(b.numpy())
    np.testing.assert_array_equal(to_np(qb), OC.int4_pack(qbo))
    c = M.grouped_gemm_w4a16(a_bf.to(dev()), qb, s7, torch.from_numpy(offsets).to(dev()), R, N,
                             swiglu=swiglu)
    ref = O.grouped_gemm(a_bf.float().numpy(), OC.int4_dequant(qbo, s7o), offsets)
    live = np.zeros(R, bool)
    for g in range(len(sizes)):
        live[offsets[g]:offsets[g] + sizes[g]] = True
    if swiglu:
        ref = O.swiglu(ref[:, :N], ref[:, N:])
    beyond, raw = error_ratios(to_np(c)[live], ref[live])
    print(f"beyond={beyond:.3e} raw={raw:.3e}")
    assert beyond <= TOL


@pytest.mark.parametrize("swiglu", [False, True])
def test_grouped_gemm_f32(swiglu):
    sizes = [30, 0, 19, 64]
    N, K = 96, 200
    note(f"gemm f32 swiglu={swiglu}")
    rng = np.random.default_rng(1)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(offsets[-1])
    a = rng.standard_normal((R, K)).astype(np.float32)
    b = (rng.standard_normal((4, 2 * N if swiglu else N, K)) / np.sqrt(K)).astype(np.float32)
    c = M.grouped_gemm_f32(torch.from_numpy(a).to(dev()), torch.from_numpy(b).to(dev()),
                           torch.from_numpy(offsets).to(dev()), R, N, swiglu=swiglu)
    ref = O.grouped_gemm(a, b, offsets)
    if swiglu:
        ref = O.swiglu(ref[:, :N], ref[:, N:])
    beyond, raw = error_ratios(to_np(c), ref, rounding=0.0)
    assert raw <= TOL


@pytest.mark.parametrize("T,k,E,cap", [
    (99, 4, 16, 20),      # some slots dropped
    (64, 10, 32, 3),      # two load batches of slots; tokens with every slot dropped
    (50, 1, 8, 0),        # one slot per token, no capacity limit
    (70, 2, 8, 0),        # the two-slot batch
    (33, 6, 12, 5),       # a partly used eight-slot batch, with drops
    (40, 8, 16, 0),       # a full eight-slot batch
])
@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32])
def test_combine(o_dtype, T, k, E, cap):
    note(f"combine {o_dtype} T={T} k={k} E={E} cap={cap}")
    d = 256
    idx = synth.random_topk(T, E, k, seed=5)
    _, offsets, ros, sor = O.dispatch(idx, E, 8, cap=cap)
    if cap == 3:
        assert np.any(np.all(ros.reshape(T, k) < 0, axis=1)), "no fully dropped token"
    R = len(sor)
    o = synth.normal((R, d), 14, "x", dtype=o_dtype)
    w = synth.uniform((T, k), 0, 1, 14, "bias")
    y = M.moe_combine(o.to(dev()), torch.from_numpy(ros).to(dev()), w.to(dev()), T, k, o_dtype)
    ref = O.combine(o.float().numpy(), ros, w.numpy(), T, k)
    if o_dtype == torch.bfloat16:
        beyond, raw = error_ratios(to_np(y), ref)
        assert beyond <= 1e-5
    else:
        beyond, raw = error_ratios(to_np(y), ref, rounding=0.0)
        assert raw <= 1e-5


def test_determinism():
    note("determinism")
    a, b, offsets, R = _gemm_case([200, 3, 77], 256, 512, 16, 15, True)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, sb = M.moe_quant_weight_fp8(b.to(dev()))
    qb = M.moe_pack_weight_fp8(qb)
    off = torch.from_numpy(offsets).to(dev())
    c1, s1 = M.grouped_gemm_fp8(qa, sa, qb, sb, off, R, 256, swiglu=True)
    c2, s2 = M.grouped_gemm_fp8(qa, sa, qb, sb, off, R, 256, swiglu=True)
    live = np.zeros(R, bool)
    live[:offsets[-1]] = True
    assert torch.equal(c1[:offsets[-1]], c2[:offsets[-1]])
    assert torch.equal(s1[:offsets[-1]], s2[:offsets[-1]])


def test_device_supported():
    """The GPU these tests run on is a gfx950: the library accepts it."""
    note("device supported")
    assert M.moe_device_supported(0)


# ------------------------------------------------ 4-bit weights on the FP8 core

def _pack_int4_reference(q, s7):
    """moe_pack_weight_int4's order written out with numpy: codes [G][N/16][KB][64][16 B]
    with lane l of block (nb, kb) holding bytes 64 kb + 16 (l // 16) .. +16 of row
    16 nb + l % 16; scales [G][N/16][KB][16]."""
    G, N, K2 = q.shape
    KB = K2 // 64
    x = q.reshape(G, N // 16, 16, KB, 4, 16)        # g, nb, r, kb, c, byte
    x = x.transpose(0, 1, 3, 4, 2, 5)               # g, nb, kb, c, r, byte (lane = 16 c + r)
    sf = s7.reshape(G, N // 16, 16, KB).transpose(0, 1, 3, 2)
    return np.ascontiguousarray(x).reshape(G, N, K2), np.ascontiguousarray(sf).reshape(G, N, KB)


def test_pack_weight_int4_permutation():
    note("pack weight int4")
    w = synth.normal((3, 256, 384), 17, "w13", std=0.02)
    q, s7 = M.moe_quant_weight_int4(w.to(dev()))
    qf, s7f = M.moe_pack_weight_int4(q, s7)
    rq, rs = _pack_int4_reference(to_np(q), to_np(s7))
    np.testing.assert_array_equal(to_np(qf), rq)
    np.testing.assert_array_equal(to_np(s7f), rs)


def _w4a8_case(sizes, N, K, m_align, seed, swiglu):
    a, b, offsets, R = _gemm_case(sizes, N, K, m_align, seed, swiglu)
    qa, sa = M.moe_quant_fp8(a.to(dev()))
    qb, s7 = M.moe_quant_weight_int4(b.to(dev()))
    qbf, s7f = M.moe_pack_weight_int4(qb, s7)
    qao, sao = OC.quant_fp8_act(a.numpy())
    cbo, s7o = OC.int4_quant_rows(b.numpy())
    np.testing.assert_array_equal(to_np(qb), OC.int4_pack(cbo))
    np.testing.assert_array_equal(to_np(s7), s7o)
    live = np.zeros(R, bool)
    for g in range(len(sizes)):
        live[offsets[g]:offsets[g] + sizes[g]] = True
    return qa, sa, qbf, s7f, qao, sao, cbo, s7o, offsets, R, live


@pytest.mark.parametrize("sizes,m_align,K", [
    ([128, 256, 64, 512, 128, 256, 64, 512], 128, 512),   # 128-row tiles
    ([0, 1, 17, 130, 300, 0], 16, 384),                     # empty, tiny, ragged groups
    ([5, 3, 9, 2, 7, 1, 4, 6, 8, 3], 8, 256),              # decode-sized groups (16-row tiles)
    ([40, 33, 50, 20], 32, 1536),                          # 32-row tiles, longer K
    ([3, 20, 40, 150], 16, 128),                           # one K block
])
@pytest.mark.parametrize("swiglu", [False, True])
def test_grouped_gemm_w4a8(sizes, m_align, K, swiglu):
    """4-bit weights (every code -7..7 occurs) expanded to e4m3 in registers on the FP8
    matrix core, promoted per block with the row scale and each channel's own scale."""
    N = 128 if swiglu else 256
    note(f"gemm w4a8 sizes={sizes} m_align={m_align} K={K} swiglu={swiglu}")
    qa, sa, qbf, s7f, qao, sao, cbo, s7o, offsets, R, live = _w4a8_case(sizes, N, K, m_align,
                                                                        61, swiglu)
    assert set(np.unique(cbo).tolist()) == set(range(-7, 8))
    off_d = torch.from_numpy(offsets).to(dev())
    ref = O.grouped_gemm_w4a8(qao, sao, cbo, s7o, offsets)
    if not swiglu:
        c = M.grouped_gemm_w4a8(qa, sa, qbf, s7f, off_d, R, N)
        beyond, raw = error_ratios(to_np(c)[live], ref[live])
        print(f"beyond={beyond:.3e} raw={raw:.3e}")
        assert beyond <= TOL, beyond
    else:
        codes, sc = M.grouped_gemm_w4a8(qa, sa, qbf, s7f, off_d, R, N, swiglu=True)
        A = OC.dequant_fp8_act(qao, sao)
        Bd = OC.int4_dequant_exact(cbo, s7o)
        sab = O.grouped_gemm(np.abs(A), np.abs(Bd), offsets)
        check_swiglu_codes(to_np(codes)[live], to_np(sc)[live], ref[live], sab[live], N)


def test_grouped_gemm_w4a8_gather():
    """GEMM1's activation gather with 4-bit weights: logical row r reads token a_rows[r] // k."""
    note("gemm w4a8 gather")
    T, k, E, N, K = 50, 2, 4, 128, 256
    idx = synth.random_topk(T, E, k, seed=4)
    counts, offsets, ros, sor = O.dispatch(idx, E, 16)
    x = synth.normal((T, K), 12, "x", dtype=torch.bfloat16)
    w = synth.normal((E, N, K), 12, "w13", std=K ** -0.5)
    qx, sx = M.moe_quant_fp8(x.to(dev()))
    qw, s7 = M.moe_quant_weight_int4(w.to(dev()))
    qwf, s7f = M.moe_pack_weight_int4(qw, s7)
    R = len(sor)
    c = M.grouped_gemm_w4a8(qx, sx, qwf, s7f, torch.from_numpy(offsets).to(dev()), R, N,
                            a_rows=torch.from_numpy(sor).to(dev()), a_row_div=k)
    qxo, sxo = OC.quant_fp8_act(x.float().numpy())
    cwo, s7o = OC.int4_quant_rows(w.numpy())
    live = sor >= 0
    A = np.zeros((R, K), np.uint8)
    sA = np.ones((R, K // 128), np.float32)
    A[live] = qxo[sor[live] // k]
    sA[live] = sxo[sor[live] // k]
    ref = O.grouped_gemm_w4a8(A, sA, cwo, s7o, offsets)
    beyond, raw = error_ratios(to_np(c)[live], ref[live])
    assert beyond <= TOL


@pytest.mark.parametrize("sizes,K", [([3, 20, 40, 150], 128), ([128, 256, 64, 512], 512)])
def test_determinism_w4a8(sizes, K):
    """Repeated 4-bit-weight SwiGLU launches give identical codes and scales (a regression
    test for the copy order the kernel's counted waits rely on: the first block's
    activation copy must be issued before the weight loads the prologue replays)."""
    note(f"determinism w4a8 sizes={sizes} K={K}")
    qa, sa, qbf, s7f, *_, offsets, R, live = _w4a8_case(sizes, 128, K, 16, 71, True)
    off = torch.from_numpy(offsets).to(dev())
    runs = [M.grouped_gemm_w4a8(qa, sa, qbf, s7f, off, R, 128, swiglu=True) for _ in range(6)]
    torch.cuda.synchronize()
    for c, s in runs[1:]:
        assert np.array_equal(to_np(c)[live], to_np(runs[0][0])[live])
        assert np.array_equal(to_np(s)[live], to_np(runs[0][1])[live])
