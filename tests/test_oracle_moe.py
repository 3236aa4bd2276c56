"""Pins for the oracle's routing, dispatch, grouped GEMM, SwiGLU, combine and
layer, against the pages' worked numbers, brute force and closed forms."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from oracle import codecs as C
import synth


# ------------------------------------------------------------------ routing

def _brute_topk(key, k):
    """Repeated arg-max with explicit loops; the first (lowest) index wins ties."""
    chosen = []
    for _ in range(k):
        best = None
        for e in range(len(key)):
            if e in chosen:
                continue
            if best is None or key[e] > key[best]:
                best = e
        chosen.append(best)
    return chosen


@pytest.mark.parametrize("ties", [False, True])
def test_topk_brute_force(ties):
    L = synth.random_logits(64, 9, seed=1, ties=ties).numpy()
    b = np.linspace(-0.01, 0.01, 9).astype(np.float32)
    if ties:
        b[:] = 0
    idx, w = O.topk_route(L, b, 3)
    for t in range(64):
        key = [float(np.float32(L[t, e] + b[e])) for e in range(9)]
        assert list(idx[t]) == _brute_topk(key, 3)
        # the chosen set is one of the k-subsets with the largest key sum
        best = max(sum(key[e] for e in s) for s in itertools.combinations(range(9), 3))
        assert math.isclose(sum(key[e] for e in idx[t]), best, rel_tol=0, abs_tol=1e-12)
        z = np.exp(np.array(key) - max(key))
        p = z / z.sum()
        np.testing.assert_allclose(w[t], p[idx[t]], rtol=1e-15)


def test_topk_k_equals_E_and_renorm():
    L = synth.random_logits(16, 6, seed=2).numpy()
    b = np.zeros(6, np.float32)
    idx, w = O.topk_route(L, b, 6)
    idx_r, w_r = O.topk_route(L, b, 6, renorm=True)
    assert all(sorted(r) == list(range(6)) for r in idx)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(w, w_r, rtol=1e-14)
    # renormalised top-k weights equal softmax over the selected keys only
    idx2, w2 = O.topk_route(L, b, 2, renorm=True)
    for t in range(16):
        sel = L[t, idx2[t]].astype(np.float64)
        e = np.exp(sel - sel.max())
        np.testing.assert_allclose(w2[t], e / e.sum(), rtol=1e-14)


def test_bias_moves_selection_and_weight():
    L = np.zeros((1, 4), np.float32)
    b = np.array([0.0, 0.0, 2.0, 0.0], np.float32)
    idx, w = O.topk_route(L, b, 1)
    assert idx[0, 0] == 2
    assert math.isclose(w[0, 0], math.exp(2) / (math.exp(2) + 3), rel_tol=1e-15)


def test_hash_route_closed_form():
    ids = np.array([0, 1, 2, 12345, 129279, 1 << 31], dtype=np.int64)
    idx, w = O.hash_route(ids, 64)
    # 2654435761 = 0x9E3779B1: its low 6 bits are 0b110001 = 49
    assert idx[0, 0] == 0 and idx[1, 0] == 49 and idx[2, 0] == (2 * 49) % 64
    for i, t in zip(ids, idx[:, 0]):
        h = 0
        for _ in range(int(i)) if i < 20 else []:
            h = (h + 2654435761) % 2 ** 32
        if i < 20:
            assert t == h % 64
        assert t == (int(i) * 2654435761 % 2 ** 32) % 64
    assert np.all(w == 1.0)


def test_capacity_pages(golden):
    ex = golden["capacity_example"]
    assert O.capacity(ex["T"], ex["k"], ex["E"], ex["factor"]) == ex["value"]
    for T, k, E in [(4096, 8, 256), (100, 2, 7), (1, 1, 3)]:
        assert O.capacity(T, k, E, 2.0) == math.ceil(T * k / E) * 2
    assert O.capacity(10, 2, 4, 0) == 0


# ----------------------------------------------------------------- dispatch

@pytest.mark.parametrize("cap", [0, 5])
@pytest.mark.parametrize("m_align", [1, 16, 128])
def test_dispatch_invariants(cap, m_align):
    T, k, E = 97, 3, 11
    idx = synth.random_topk(T, E, k, seed=3, skew=1.2)
    counts, offsets, ros, sor = O.dispatch(idx, E, m_align, cap)
    flat = idx.ravel()
    # brute-force histogram
    assert [int(sum(1 for v in flat if v == e)) for e in range(E)] == list(counts)
    assert counts.sum() == T * k
    assert offsets[0] == 0 and np.all(offsets % m_align == 0)
    kept = np.minimum(counts, cap) if cap else counts
    np.testing.assert_array_equal(np.diff(offsets), -(-kept // m_align) * m_align)
    # stable order: the kept slots of each expert in increasing slot order
    order = np.argsort(flat, kind="stable")
    pos = 0
    for e in range(E):
        slots = order[pos:pos + counts[e]]
        pos += counts[e]
        for r, s in enumerate(slots):
            if cap and r >= cap:
                assert ros[s] == -1
            else:
                assert ros[s] == offsets[e] + r
                assert sor[offsets[e] + r] == s
        for r in range(kept[e], offsets[e + 1] - offsets[e]):
            assert sor[offsets[e] + r] == -1
    # bijection between kept slots and non-padding rows
    live = sor[sor >= 0]
    assert len(live) == len(set(live.tolist())) == kept.sum()
    assert np.all(sor[offsets[E]:] == -1)
    assert len(sor) == T * k + E * (m_align - 1)


@pytest.mark.parametrize("cap", [1, 4, 40])
def test_dispatch_masked_layout(cap):
    """Fixed-capacity layout: expert e's rows are [e C, e C + C) whatever its load, filled
    by its first C slots in slot order (numpy's stable argsort decides the order here, a
    different route from the oracle's slot loop); the same ranks and drops as the
    contiguous dispatch with that capacity."""
    T, k, E = 61, 3, 9
    idx = synth.random_topk(T, E, k, seed=7, skew=1.3)
    counts, ros, sor = O.dispatch_masked(idx, E, cap)
    flat = idx.ravel()
    assert [int(np.sum(flat == e)) for e in range(E)] == list(counts)
    order = np.argsort(flat, kind="stable")
    want_ros = np.full(T * k, -1, np.int64)
    start = np.concatenate([[0], np.cumsum(counts)])
    for e in range(E):
        for r, s_ in enumerate(order[start[e]:start[e + 1]]):
            if r < cap:
                want_ros[s_] = e * cap + r
    np.testing.assert_array_equal(ros, want_ros)
    assert len(sor) == E * cap
    for row in range(E * cap):
        s_ = sor[row]
        assert (s_ == -1) if row % cap >= min(counts[row // cap], cap) else ros[s_] == row
    # relation to the contiguous layout with the same capacity: same kept slots, each
    # expert's block moved from offsets[e] to e * C
    c2, offsets, ros2, _ = O.dispatch(idx, E, 1, cap)
    np.testing.assert_array_equal(counts, c2)
    kept = ros2 >= 0
    np.testing.assert_array_equal(ros >= 0, kept)
    e_of = flat[kept]
    np.testing.assert_array_equal(ros[kept] - e_of * cap, ros2[kept] - offsets[e_of])


# ------------------------------------------------------------- grouped GEMM

def _frac(x):
    return Fraction(float(x))


def test_grouped_gemm_fp8_exact_fractions():
    rng = np.random.default_rng(9)
    sizes = [3, 0, 5]
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    R, N, K = offsets[-1], 128, 256
    qA = rng.integers(0, 256, (R, K)).astype(np.uint8)
    qA[(qA & 0x7F) == 0x7F] = 0x01                    # no NaN codes
    qB = rng.integers(0, 256, (3, N, K)).astype(np.uint8)
    qB[(qB & 0x7F) == 0x7F] = 0x02
    sA = (rng.random((R, 2)) + 0.5).astype(np.float32)
    sB = (rng.random((3, 1, 2)) + 0.5).astype(np.float32)
    Cm = O.grouped_gemm_fp8(qA, sA, qB, sB, offsets)
    tab = C.e4m3_decode_table()
    for r in range(R):
        g = int(np.searchsorted(offsets, r, side="right") - 1)
        for n in (0, 1, 77, 127):
            total = Fraction(0)
            for kb in range(2):
                part = Fraction(0)
                for kk in range(kb * 128, kb * 128 + 128):
                    part += _frac(tab[qA[r, kk]]) * _frac(tab[qB[g, n, kk]])
                total += _frac(sA[r, kb]) * _frac(sB[g, 0, kb]) * part
            assert abs(float(total) - Cm[r, n]) <= 1e-12 * max(1.0, abs(float(total)))


def test_grouped_gemm_integer_codes_exact(golden):
    """Unit scales and small-integer codes give exact integer results; groups follow
    the page's example group sizes and must match an integer per-group loop."""
    sizes = golden["deepgemm_group_sizes"]["value"]
    rng = np.random.default_rng(10)
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    R, N, K = offsets[-1], 128, 128
    ints = np.array([-4, -3, -2, -1, 0, 1, 2, 3, 4])
    a_int = rng.choice(ints, (R, K))
    b_int = rng.choice(ints, (len(sizes), N, K))
    qA = C.e4m3_encode(a_int.astype(np.float32))
    qB = C.e4m3_encode(b_int.astype(np.float32))
    Cm = O.grouped_gemm_fp8(qA, np.ones((R, 1), np.float32), qB,
                            np.ones((len(sizes), 1, 1), np.float32), offsets)
    for g in range(len(sizes)):
        lo, hi = offsets[g], offsets[g + 1]
        ref = a_int[lo:hi].astype(np.int64) @ b_int[g].astype(np.int64).T
        np.testing.assert_array_equal(Cm[lo:hi], ref)


def test_grouped_equals_concatenation():
    """Y = Concat(E_1(T_1), ..., E_E(T_E)) -- the grouped product equals running
    each group separately (discosf.com sec. 2.1)."""
    rng = np.random.default_rng(11)
    sizes = [4, 7, 0, 2]
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    A = rng.standard_normal((offsets[-1], 64))
    B = rng.standard_normal((4, 32, 64))
    Cm = O.grouped_gemm(A, B, offsets)
    parts = [torch.from_numpy(A[offsets[g]:offsets[g + 1]]) @ torch.from_numpy(B[g]).T
             for g in range(4)]
    np.testing.assert_allclose(Cm, torch.cat(parts).numpy(), rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ SwiGLU

def test_silu_special_values():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 800.0, -800.0])
    s = O.silu(z)
    assert s[0] == 0.0
    assert math.isclose(s[1], 1 / (1 + math.exp(-1)), rel_tol=1e-15)
    assert math.isclose(s[1] - s[2], 1.0, rel_tol=1e-15)   # silu(z) - silu(-z) = z
    assert math.isclose(s[3], 40.0, rel_tol=1e-15) and abs(s[4]) < 1e-15
    assert s[5] == 800.0 and s[6] == 0.0


# ------------------------------------------------------------------- layer

def _fp32_experts(E, d, I, seed):
    w = synth.Workload("t", T=1, d=d, E=E, k=1, I=I, mode="fp32", seed=seed)
    return (synth.expert_weights(w, "w13").numpy(), synth.expert_weights(w, "w2").numpy())


def test_layer_single_expert_is_dense_ffn():
    T, d, I = 9, 128, 64
    x = synth.normal((T, d), 0, "x").numpy()
    w13, w2 = _fp32_experts(1, d, I, 0)
    out = O.layer_forward("fp32", x, E=1, k=1, I=I, w_router=np.zeros((1, d), np.float32),
                          bias=np.zeros(1, np.float32), experts=(w13, w2))
    xt = torch.from_numpy(x).double()
    g = xt @ torch.from_numpy(w13[0, :I]).double().T
    u = xt @ torch.from_numpy(w13[0, I:]).double().T
    ref = (torch.nn.functional.silu(g) * u) @ torch.from_numpy(w2[0]).double().T
    np.testing.assert_allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_layer_k_equals_E_is_soft_moe():
    """With k = E every expert is used with its full softmax weight, which is the
    dense soft-MoE sum over all experts (mooersco.com sec. 2.3)."""
    T, d, E, I = 12, 128, 4, 32
    x = synth.normal((T, d), 1, "x").numpy()
    wr = synth.normal((E, d), 1, "w_gate_router", std=d ** -0.5).numpy()
    b = synth.uniform((E,), -0.01, 0.01, 1, "bias").numpy()
    w13, w2 = _fp32_experts(E, d, I, 1)
    out = O.layer_forward("fp32", x, E=E, k=E, I=I, w_router=wr, bias=b, experts=(w13, w2))
    xt = torch.from_numpy(x).double()
    logits = (xt @ torch.from_numpy(wr).double().T).float()
    p = torch.softmax((logits + torch.from_numpy(b)).double(), dim=1)
    ys = []
    for e in range(E):
        g = xt @ torch.from_numpy(w13[e, :I]).double().T
        u = xt @ torch.from_numpy(w13[e, I:]).double().T
        ys.append((torch.nn.functional.silu(g) * u) @ torch.from_numpy(w2[e]).double().T)
    ref = torch.einsum("te,etd->td", p, torch.stack(ys))
    np.testing.assert_allclose(out["y"], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_layer_token_permutation_invariance():
    T, d, E, k, I = 20, 128, 5, 2, 32
    x = synth.normal((T, d), 2, "x").numpy()
    wr = synth.normal((E, d), 2, "w_gate_router", std=d ** -0.5).numpy()
    b = synth.uniform((E,), -0.01, 0.01, 2, "bias").numpy()
    w13, w2 = _fp32_experts(E, d, I, 2)
    perm = np.random.default_rng(0).permutation(T)
    a = O.layer_forward("fp32", x, E=E, k=k, I=I, w_router=wr, bias=b, experts=(w13, w2))
    bb = O.layer_forward("fp32", x[perm], E=E, k=k, I=I, w_router=wr, bias=b,
                         experts=(w13, w2))
    np.testing.assert_array_equal(a["y"][perm], bb["y"])


def test_layer_fp8_matches_dequantised_fp32_layer():
    """The fp8 layer equals the fp32 layer run on the dequantised weights and the
    dequantised (requantised) activations: checks that quantisation enters only
    where the method puts it."""
    T, d, E, k, I = 16, 256, 4, 2, 128
    x = synth.normal((T, d), 3, "x", dtype=torch.bfloat16).float().numpy()
    wr = synth.normal((E, d), 3, "w_gate_router", std=d ** -0.5,
                      dtype=torch.bfloat16).float().numpy()
    b = synth.uniform((E,), -0.01, 0.01, 3, "bias").numpy()
    w13, w2 = _fp32_experts(E, d, I, 3)
    q13, s13 = C.quant_fp8_weight(w13)
    q2, s2 = C.quant_fp8_weight(w2)
    out = O.layer_forward("fp8", x, E=E, k=k, I=I, w_router=wr, bias=b,
                          experts=(q13, s13, q2, s2))
    # independent restatement with torch fp64 and torch's e4m3 cast
    qx, sx = C.quant_fp8_act(x)
    xd = torch.from_numpy(C.dequant_fp8_act(qx, sx))
    W13 = torch.from_numpy(C.dequant_fp8_weight(q13, s13))
    W2 = torch.from_numpy(C.dequant_fp8_weight(q2, s2))
    y = torch.zeros(T, d, dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            e = int(out["idx"][t, j])
            gu = W13[e] @ xd[t]
            h = (torch.nn.functional.silu(gu[:I]) * gu[I:]).float()
            hb = h.view(1, I // 128, 128)
            s = hb.abs().amax(dim=2) / 448.0
            hq = (hb / s[:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).double()
            hd = (hq * s.double()[:, :, None]).view(I)
            y[t] += out["w"][t, j] * (W2[e] @ hd)
    np.testing.assert_allclose(out["y"], y.numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ combine

def _combine_sparse(o, ros, w, T, k):
    """y = S o with S [T, rows] the sparse gate matrix, S[t, row(t, j)] = w[t, j] for
    kept slots: the combine written as one sparse-dense product (scipy), a different
    route from the oracle's per-slot loop."""
    import scipy.sparse as sp
    ros = np.asarray(ros).reshape(T * k)
    w = np.asarray(w, np.float64).reshape(T * k)
    keep = ros >= 0
    tok = np.repeat(np.arange(T), k)[keep]
    S = sp.csr_matrix((w[keep], (tok, ros[keep])), shape=(T, o.shape[0]))
    return np.asarray(S @ np.asarray(o, np.float64))


def _combine_pins_hold(fn) -> bool:
    """Whether a combine implementation ``fn(o, row_of_slot, w, T, k)`` meets every pin:
    the worked integer example, and agreement with the sparse product on random cases
    with dropped slots, k = 1 and k = E (y = sum over the top-k of G(x)_i E_i(x),
    discosf.com sec. 2.1)."""
    # worked example: T = 3 tokens, k = 2, d = 3; dyadic weights, so every sum is exact.
    # token 0 -> rows 2 (w 0.5) and 0 (w 0.25); token 1 -> row 1 (w 1), slot 1 dropped;
    # token 2 -> both slots dropped.
    o = np.array([[4.0, -8.0, 12.0], [1.0, 2.0, 3.0], [-2.0, 6.0, 10.0], [100.0, 100.0, 100.0]])
    ros = np.array([2, 0, 1, -1, -1, -1], np.int32)
    w = np.array([[0.5, 0.25], [1.0, 0.5], [0.75, 0.125]])
    want = np.array([[-1.0 + 1.0, 3.0 - 2.0, 5.0 + 3.0],   # 0.5*row2 + 0.25*row0
                     [1.0, 2.0, 3.0],
                     [0.0, 0.0, 0.0]])
    try:
        if not np.array_equal(fn(o, ros, w, 3, 2), want):
            return False
        rng = np.random.default_rng(17)
        for T, k, E, cap in ((13, 3, 5, 6), (9, 1, 4, 0), (7, 4, 4, 0), (11, 2, 3, 2)):
            idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
            _, offsets, r, sor = O.dispatch(idx, E, 4, cap)
            oo = rng.standard_normal((len(sor), 6))
            ww = rng.uniform(0.1, 1.0, (T, k))
            got = fn(oo, r, ww, T, k)
            if got.shape != (T, 6) or not np.allclose(got, _combine_sparse(oo, r, ww, T, k),
                                                      rtol=1e-13, atol=1e-13):
                return False
    except (IndexError, ValueError):
        return False
    return True


def test_combine_pins():
    assert _combine_pins_hold(O.combine)


def test_combine_pins_catch_planted_mistakes():
    """Each plausible slip in a combine (transposed slot order, weights read by the wrong
    index, a dropped slot's -1 used as a row) fails the pins above."""
    def transposed_slots(o, ros, w, T, k):
        return O.combine(o, np.asarray(ros).reshape(k, T).T.ravel(), w, T, k)

    def weight_index(o, ros, w, T, k):
        return O.combine(o, ros, np.asarray(w).reshape(T, k)[:, ::-1], T, k)

    def drop_as_row(o, ros, w, T, k):
        o = np.asarray(o, np.float64)
        r = np.asarray(ros).reshape(T, k)
        wk = np.asarray(w, np.float64).reshape(T, k)
        return sum(wk[:, j:j + 1] * o[r[:, j]] for j in range(k))

    for bad in (transposed_slots, weight_index, drop_as_row):
        assert not _combine_pins_hold(bad), bad.__name__


def test_layer_output_is_combine_of_expert_rows():
    """layer_forward's y equals oracle.combine over its own expert rows, so the layer's
    weighted sum and the pinned combine are one operation."""
    T, d, E, k, I = 24, 128, 6, 3, 64
    x = synth.normal((T, d), 4, "x").numpy()
    wr = synth.normal((E, d), 4, "w_gate_router", std=d ** -0.5).numpy()
    b = synth.uniform((E,), -0.01, 0.01, 4, "bias").numpy()
    w13, w2 = _fp32_experts(E, d, I, 4)
    out = O.layer_forward("fp32", x, E=E, k=k, I=I, w_router=wr, bias=b, experts=(w13, w2),
                          m_align=4, cap_factor=1.0)
    ros = out["row_of_slot"]
    assert np.any(ros < 0)                       # the capacity dropped some slots
    o_rows = np.zeros((len(out["slot_of_row"]), d))
    for s, v in out["o_by_slot"].items():
        o_rows[ros[s]] = v
    np.testing.assert_allclose(out["y"], O.combine(o_rows, ros, out["w"], T, k),
                               rtol=1e-14, atol=1e-14)


def test_grouped_gemm_w4a8_exact_fractions():
    """The 4-bit-weight grouped GEMM against exact rational arithmetic on random codes
    (every code -7..7) and scales: C = sum_kb sA * s7 * sum_k e4m3(qA) * q."""
    rng = np.random.default_rng(13)
    G, N, K = 2, 3, 256
    offsets = np.array([0, 2, 5])
    qA = rng.integers(0, 256, (5, K)).astype(np.uint8)
    qA[(qA & 0x7F) == 0x7F] = 0x11                     # no NaN codes
    sA = rng.uniform(0.01, 2, (5, K // 128)).astype(np.float32)
    q = rng.integers(-7, 8, (G, N, K)).astype(np.int8)
    s7 = rng.uniform(0.001, 0.1, (G, N, K // 128)).astype(np.float32)
    got = O.grouped_gemm_w4a8(qA, sA, q, s7, offsets)
    dec = C.e4m3_decode_table()
    for g in range(G):
        for r in range(offsets[g], offsets[g + 1]):
            for n in range(N):
                tot = Fraction(0)
                for kb in range(K // 128):
                    part = sum(Fraction(float(dec[qA[r, k]])) * int(q[g, n, k])
                               for k in range(kb * 128, kb * 128 + 128))
                    tot += Fraction(float(sA[r, kb])) * Fraction(float(s7[g, n, kb])) * part
                assert math.isclose(got[r, n], float(tot), rel_tol=1e-12, abs_tol=1e-12)


def test_layer_w4a8_matches_restatement():
    """The 4-bit-weight layer on the FP8 path equals the same maths written with torch: the
    weights q * s7, the activations and h through torch's own e4m3 cast at 1x128 scales."""
    T, d, E, k, I = 16, 256, 4, 2, 128
    x = synth.normal((T, d), 6, "x", dtype=torch.bfloat16).float().numpy()
    wr = synth.normal((E, d), 6, "w_gate_router", std=d ** -0.5,
                      dtype=torch.bfloat16).float().numpy()
    b = synth.uniform((E,), -0.01, 0.01, 6, "bias").numpy()
    w13, w2 = _fp32_experts(E, d, I, 6)
    c13, s13 = C.int4_quant_rows(w13)
    c2, s2 = C.int4_quant_rows(w2)
    out = O.layer_forward("w4a8", x, E=E, k=k, I=I, w_router=wr, bias=b,
                          experts=(c13, s13, c2, s2))

    def q1x128(v):
        vb = v.view(v.shape[0], -1, 128)
        s = vb.abs().amax(dim=2) / 448.0
        s = torch.where(s == 0, torch.ones_like(s), s)
        qv = (vb / s[:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).double()
        return (qv * s.double()[:, :, None]).view(v.shape)

    def w_exact(c, s7):
        ct = torch.from_numpy(c.astype(np.float64))
        return ct * torch.from_numpy(s7.astype(np.float64)).repeat_interleave(128, dim=-1)

    xd = q1x128(torch.from_numpy(x))
    W13, W2 = w_exact(c13, s13), w_exact(c2, s2)
    y = torch.zeros(T, d, dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            e = int(out["idx"][t, j])
            gu = W13[e] @ xd[t]
            h = (torch.nn.functional.silu(gu[:I]) * gu[I:]).float()
            hd = q1x128(h[None])[0]
            y[t] += out["w"][t, j] * (W2[e] @ hd)
    np.testing.assert_allclose(out["y"], y.numpy(), rtol=1e-12, atol=1e-12)
