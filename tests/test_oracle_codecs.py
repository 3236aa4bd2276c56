"""Pins for the oracle's number formats, against the pages' figures, exhaustive
enumeration and torch's independent CPU casts."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs as C


def test_e4m3_table_shape_and_extremes(golden):
    t = C.e4m3_decode_table()
    finite = t[np.isfinite(t)]
    assert finite.size == 254                       # 256 codes minus the two NaNs
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert finite.max() == golden["e4m3_max"]["value"] == 448.0
    assert finite.min() == -448.0
    assert t[0x01] == 2.0 ** -9                      # smallest subnormal
    assert t[0x08] == 2.0 ** -6                      # smallest normal
    assert t[0x38] == 1.0                            # exponent field 7 = bias
    # 253 distinct values (+0 and -0 coincide)
    assert np.unique(finite).size == 253


def test_e4m3_roundtrip_every_code():
    t = C.e4m3_decode_table()
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    back = C.e4m3_encode(t[codes].astype(np.float32))
    np.testing.assert_array_equal(back, codes)


def test_e4m3_ties_go_to_even_and_saturate():
    t = C.e4m3_decode_table()
    pos = np.sort(np.unique(t[np.isfinite(t) & (t >= 0)]))
    mids = (pos[:-1] + pos[1:]) / 2                  # exact midpoints (fp32 exact)
    codes = C.e4m3_encode(mids.astype(np.float32))
    for m, c in zip(mids, codes):
        lo = pos[pos < m].max()
        hi = pos[pos > m].min()
        clo = C.e4m3_encode(np.float32(lo))
        chi = C.e4m3_encode(np.float32(hi))
        assert c in (clo, chi)
        assert int(c) % 2 == 0                       # even mantissa wins the tie
    # beyond the largest finite value: saturate, never NaN
    big = np.array([448.0, 460.0, 464.0, 1e6, -1e30], dtype=np.float32)
    np.testing.assert_array_equal(C.e4m3_encode(big), [0x7E, 0x7E, 0x7E, 0x7E, 0xFE])


def test_e4m3_matches_torch_cast():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(300_000) * np.exp2(rng.integers(-14, 9, 300_000))
    v = np.clip(v, -448, 448).astype(np.float32)
    mine = C.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mine, ref)


def test_bf16_matches_torch_and_definition():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal(300_000) * np.exp2(rng.integers(-130, 120, 300_000))).astype(np.float32)
    mine = C.bf16_round(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(mine, ref)
    # worked ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1)
    assert C.bf16_round(np.float32(1 + 2 ** -8)) == 1.0
    assert C.bf16_round(np.float32(1 + 3 * 2 ** -8)) == np.float32(1 + 2 ** -6)


def test_quant_act_block_rules():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 384)).astype(np.float32)
    x[2, 128:256] = 0.0                              # an all-zero block
    q, s = C.quant_fp8_act(x)
    assert q.shape == (6, 384) and s.shape == (6, 3) and s.dtype == np.float32
    assert s[2, 1] == 1.0 and np.all(q[2, 128:256] == 0)
    for r in range(6):
        for b in range(3):
            blk = x[r, b * 128:(b + 1) * 128]
            if not blk.any():
                continue
            j = np.argmax(np.abs(blk))
            # the block's largest element lands exactly on +-448
            assert C.e4m3_decode(q[r, b * 128 + j]) == math.copysign(448.0, blk[j])
            assert s[r, b] == np.float32(np.float32(np.abs(blk).max()) / np.float32(448))
    # error bound: half an e4m3 spacing (2^-4 relative for normals, 2^-10 * s below)
    deq = C.dequant_fp8_act(q, s)
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, np.repeat(s, 128, axis=1) * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_quant_act_matches_torch_pipeline():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((16, 512)) * 3).astype(np.float32)
    q, s = C.quant_fp8_act(x)
    xt = torch.from_numpy(x).view(16, 4, 128)
    amax = xt.abs().amax(dim=2)
    st = amax / 448.0
    qt = (xt / st[:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    np.testing.assert_array_equal(q, qt.reshape(16, 512).numpy())
    np.testing.assert_array_equal(s, st.numpy())


def test_quant_weight_blocks():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((2, 256, 384)).astype(np.float32)
    q, s = C.quant_fp8_weight(w)
    assert s.shape == (2, 2, 3)
    for g in range(2):
        for nb in range(2):
            for kb in range(3):
                blk = w[g, nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
                assert s[g, nb, kb] == np.float32(np.abs(blk).max()) / np.float32(448)
                qb = q[g, nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
                assert np.sum(np.abs(C.e4m3_decode(qb)) == 448.0) >= 1
    # transposing the block grid must move the scales with it
    q2, s2 = C.quant_fp8_weight(np.ascontiguousarray(np.swapaxes(w[:, :, :256], 1, 2)))
    np.testing.assert_array_equal(s2, np.swapaxes(s[:, :, :2], 1, 2))


def test_int4_block_rules(golden):
    rng = np.random.default_rng(8)
    w = rng.standard_normal((2, 5, 256)).astype(np.float32)
    q, s7 = C.int4_quant_rows(w)
    levels = golden["int4_levels"]["value"]
    assert q.min() >= -levels and q.max() <= levels
    for g in range(2):
        for n in range(5):
            for b in range(2):
                blk = w[g, n, b * 128:(b + 1) * 128]
                j = np.argmax(np.abs(blk))
                assert abs(int(q[g, n, b * 128 + j])) == levels
                assert s7[g, n, b] == np.float32(np.float32(np.abs(blk).max()) / np.float32(7))
    deq = C.int4_dequant(q, s7)
    scale = np.repeat(s7 * 7, 128, axis=2)
    err = np.abs(deq.astype(np.float64) - w)
    assert np.all(err <= scale / 14 + np.abs(w) * 2.0 ** -7 + 1e-7)
    packed = C.int4_pack(q)
    assert packed.shape == (2, 5, 128)
    # unpack byte by byte with the layout's rule, independently of the packer
    flat = packed.reshape(-1, 128)
    ref = q.reshape(-1, 256)
    for row in range(flat.shape[0]):
        for byte in range(128):
            p, b = divmod(byte, 4)
            v = int(flat[row, byte])
            for nib, k in ((v & 0xF, 8 * p + b), (v >> 4, 8 * p + 4 + b)):
                val = -(nib & 7) if nib & 8 else nib & 7
                assert val == ref[row, k]


def test_int4_pack_layout_example():
    # codes 1, -2, 3, -4, 5, -6, 7, 0 -> nibbles 1, A, 3, C, 5, E, 7, 0 -> bytes 51 EA 73 0C
    q = np.array([[1, -2, 3, -4, 5, -6, 7, 0]], np.int8)
    assert C.int4_pack(q).tolist() == [[0x51, 0xEA, 0x73, 0x0C]]
    with pytest.raises(ValueError):
        C.int4_pack(np.full((1, 8), -8, np.int8))


def test_fp4_bytes_example(golden):
    ex = golden["fp4_bytes_example"]
    n = ex["shape"][0] * ex["shape"][1]
    assert round(n * 2 / 2 ** 20) == ex["fp16_MiB"]
    assert round(n * 0.5 / 2 ** 20) == ex["fp4_MiB"]


def _int4_dequant_by_torch(q, s7):
    """bf16(fl32(q * s7)) with torch's fp32 product and torch's own RNE bf16 cast."""
    qt = torch.from_numpy(np.asarray(q, np.int8).astype(np.float32))
    G, N, K = qt.shape
    st = torch.from_numpy(np.asarray(s7, np.float32)).repeat_interleave(128, dim=2)
    return (qt * st).to(torch.bfloat16).to(torch.float32).numpy().reshape(G, N, K)


def test_int4_dequant_exact_every_code():
    """Exact pin of the dequantised int4 weight bf16(fl32(q * s7)) (tqpw.cn sec. 3.1, read
    as the bf16 value the matrix product consumes): every code -7..7 against a sweep of
    stored scales (random mantissas over many binades, powers of two, values whose
    products sit on bf16 rounding ties), compared bit for bit with torch's casts."""
    rng = np.random.default_rng(23)
    codes = np.tile(np.arange(-7, 8, dtype=np.int8), 9)[:128]
    s = np.concatenate([
        rng.uniform(1.0, 2.0, 300) * np.exp2(rng.integers(-30, 10, 300)),
        np.exp2(np.arange(-20, 5, dtype=np.float64)),
        1.0 + np.arange(1, 64) * 2.0 ** -8,          # q * s7 lands on bf16 ties for odd q
        (1.0 + 2.0 ** -7) / 3.0 * np.ones(4),
    ]).astype(np.float32)
    q = np.broadcast_to(codes, (len(s), 128))[None].copy()
    s7 = s[None, :, None]
    got = C.int4_dequant(q, s7)
    want = _int4_dequant_by_torch(q, s7)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    # a different rounding order (bf16 scale times code) disagrees on this sweep
    alt = (torch.from_numpy(s).to(torch.bfloat16).float()[:, None] *
           torch.from_numpy(codes.astype(np.float32))[None, :]).numpy()[None]
    assert np.any(alt != want)


def test_int4_quant_dequant_roundtrip_exact_codes():
    """Weights that are exact multiples of their block's s7 survive quantisation: the codes
    come back unchanged and the dequantised weight is bf16 of that multiple."""
    rng = np.random.default_rng(29)
    q0 = rng.integers(-7, 8, (2, 3, 256)).astype(np.int8)
    q0[:, :, 5] = 7                               # every block holds its maximum code
    q0[:, :, 133] = -7
    s7 = np.float32(2.0 ** -5)
    w = q0.astype(np.float32) * s7                # exact in fp32
    q, s7o = C.int4_quant_rows(w)
    np.testing.assert_array_equal(q, q0)
    assert np.all(s7o == s7)
    np.testing.assert_array_equal(C.int4_dequant(q, s7o), w)


def test_int4_codes_exact_as_e4m3_every_code():
    """Each of the 15 codes -7..7 the lecture's 4-bit rule produces (tqpw.cn sec. 3.1) is an
    exact e4m3 value: encoding and decoding returns the integer, so the FP8 matrix core
    multiplies them exactly.  Also their e4m3 bit patterns, from the format's definition
    (sign, exponent with bias 7, 3 mantissa bits)."""
    q = np.arange(-7, 8, dtype=np.float64)
    codes = C.e4m3_encode(q)
    np.testing.assert_array_equal(C.e4m3_decode(codes), q)
    # 1 = 1.0 x 2^0 -> exponent field 7; 3 = 1.5 x 2^1; 5 = 1.25 x 2^2; 7 = 1.75 x 2^2
    want = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 5: 0x4A, 6: 0x4C, 7: 0x4E}
    for v, c in zip(q.astype(int), codes):
        assert int(c) == (want[abs(v)] | (0x80 if v < 0 else 0)), (v, hex(c))


def test_int4_dequant_exact_relations():
    """The exact 4-bit weight q * s7 against brute-force products of Python floats (exact:
    3-bit integers times fp32 values fit an fp64 mantissa), and the W4A16 weight is its
    fp32 rounding rounded to bf16."""
    rng = np.random.default_rng(31)
    q = rng.integers(-7, 8, (2, 3, 256)).astype(np.int8)
    s7 = (rng.uniform(0.5, 2.0, (2, 3, 2)) * 2.0 ** rng.integers(-12, 3, (2, 3, 2))).astype(np.float32)
    ex = C.int4_dequant_exact(q, s7)
    for g in range(2):
        for n in range(3):
            for k in range(256):
                assert ex[g, n, k] == int(q[g, n, k]) * float(s7[g, n, k // 128])
    np.testing.assert_array_equal(C.bf16_round(ex.astype(np.float32)), C.int4_dequant(q, s7))
