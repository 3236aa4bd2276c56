"""Number formats used by the layer, written from their definitions (oracle side).

* e4m3 ("fn" variant): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 is subnormal; the all-ones pattern S.1111.111 is NaN, so the
  largest finite magnitude is 1.75 * 2^8 = 448 -- the clamp bound the MegaMoE
  article gives for e4m3 quantisation (discosf.com, sec. 3.3).
* bf16: the upper half of an fp32, rounded to nearest, ties to even (the article
  insists on RNE rather than truncation for the bf16 output, sec. 3.3).
* int4 block weights: round(w / blockmax * 7), the DeepSeek-V4 lecture's
  block-wise 4-bit formula (tqpw.cn, sec. 3.1).

All arithmetic here is numpy fp64 or IEEE fp32 (numpy float32 ops are correctly
rounded), never a copy of the HIP kernels' bit tricks.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_E4M3_MIN_NORMAL = 2.0 ** -6
_E4M3_SUB_QUANTUM = 2.0 ** -9


def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 e4m3 codes as fp64 (NaN for 0x7F and 0xFF)."""
    tab = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            tab[c] = np.nan
        elif e == 0:
            tab[c] = sign * m * _E4M3_SUB_QUANTUM          # m/8 * 2^(1-7)
        else:
            tab[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


_TABLE = e4m3_decode_table()


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """Exact floor(log2(a)) for a > 0 (0 -> a huge negative value), via frexp."""
    m, ex = np.frexp(np.where(a > 0, a, np.float64(2.0) ** -1074))
    return (ex - 1).astype(np.float64)


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """Saturating round-to-nearest-even fp32 -> e4m3 code (uint8).

    |v| is clamped to 448 first, as in x_fp8 = clamp(round(x/scale), -448, 448)
    (discosf.com, sec. 3.3); subnormals are kept; NaN never appears for finite v.
    The sign bit of v is kept, so values that round to zero keep their sign.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: non-finite input")
    a = np.minimum(np.abs(v), E4M3_MAX)
    # spacing of representable values around a: 2^(e-3) in binade [2^e, 2^(e+1)),
    # 2^-9 below the smallest normal 2^-6
    e = _floor_log2(a)
    e = np.maximum(e, -6.0)
    quantum = np.exp2(e - 3.0)
    n = np.rint(a / quantum)                 # numpy rint rounds half to even
    r = n * quantum                          # exact in fp64
    # value -> code
    sub = r < _E4M3_MIN_NORMAL
    code = np.zeros(a.shape, dtype=np.int64)
    code[sub] = np.rint(r[sub] / _E4M3_SUB_QUANTUM).astype(np.int64)
    rn = r[~sub]
    en = _floor_log2(rn)
    mant = np.rint((rn / np.exp2(en) - 1.0) * 8.0).astype(np.int64)
    code[~sub] = ((en.astype(np.int64) + 7) << 3) | mant
    neg = np.signbit(v)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


def bf16_round(v) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns float32 values.

    bf16 keeps fp32's 8-bit exponent and 7 stored mantissa bits, so the spacing in
    binade [2^e, 2^(e+1)) is 2^(e-7) (2^-133 for fp32 subnormals).
    """
    x = np.asarray(v, dtype=np.float32).astype(np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_round: non-finite input")
    a = np.abs(x)
    e = _floor_log2(a)
    e = np.maximum(e, -126.0)
    quantum = np.exp2(e - 7.0)
    r = np.rint(a / quantum) * quantum
    return np.copysign(r, x).astype(np.float32)


# ----------------------------------------------------------------- fp8 blocks

def _check_blocks(n: int, what: str):
    if n % 128:
        raise ValueError(f"{what} must be a multiple of 128, got {n}")


def quant_fp8_act(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-row 1x128 e4m3 quantisation of activations [R, K].

    For every row r and 128-column block c: amax = max |x| over the block,
    s = fl32(amax / 448) (s = 1 when amax = 0), q = e4m3(fl32(x / s)).
    Fine-grained (not per-tensor) scaling, as DeepGEMM's release notes describe
    (qidao123.com, day 3); the clamp/round step is discosf.com sec. 3.3.
    Returns codes uint8 [R, K] and scales float32 [R, K/128].
    """
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    _check_blocks(K, "K")
    xb = x.reshape(R, K // 128, 128)
    amax = np.max(np.abs(xb), axis=2)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    scaled = (xb / s[:, :, None]).astype(np.float32)
    return e4m3_encode(scaled).reshape(R, K), s


def dequant_fp8_act(q, s) -> np.ndarray:
    R, K = q.shape
    return (e4m3_decode(q).reshape(R, K // 128, 128) * np.asarray(s, np.float64)[:, :, None]
            ).reshape(R, K)


def quant_fp8_weight(w) -> tuple[np.ndarray, np.ndarray]:
    """128x128 block e4m3 quantisation of weights [G, N, K] (K contiguous).

    Same scale/round rule as the activations but one scale per 128x128 block:
    returns codes uint8 [G, N, K] and scales float32 [G, N/128, K/128].
    """
    w = np.asarray(w, dtype=np.float32)
    G, N, K = w.shape
    _check_blocks(N, "N")
    _check_blocks(K, "K")
    wb = w.reshape(G, N // 128, 128, K // 128, 128)
    amax = np.max(np.abs(wb), axis=(2, 4))
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    scaled = (wb / s[:, :, None, :, None]).astype(np.float32)
    return e4m3_encode(scaled).reshape(G, N, K), s


def dequant_fp8_weight(q, s) -> np.ndarray:
    G, N, K = q.shape
    v = e4m3_decode(q).reshape(G, N // 128, 128, K // 128, 128)
    return (v * np.asarray(s, np.float64)[:, :, None, :, None]).reshape(G, N, K)


# ------------------------------------------------------------- int4 blocks

def int4_quant_rows(w) -> tuple[np.ndarray, np.ndarray]:
    """Block-wise 4-bit weights with per-channel 1x128 blocks (tqpw.cn, sec. 3.1).

    For each output channel n and 128-wide K block: scale = max |w| over the block
    (1 when the block is all zero); q = round(fl32(fl32(w/scale) * 7)) in [-7, 7]
    (ties to even); the stored scale is s7 = fl32(scale / 7).
    Returns codes int8 [G, N, K] (unpacked) and s7 float32 [G, N, K/128].
    """
    w = np.asarray(w, dtype=np.float32)
    G, N, K = w.shape
    _check_blocks(K, "K")
    wb = w.reshape(G, N, K // 128, 128)
    amax = np.max(np.abs(wb), axis=3)
    amax = np.where(amax == 0, np.float32(1.0), amax).astype(np.float32)
    t = (wb / amax[:, :, :, None]).astype(np.float32)
    t = (t * np.float32(7.0)).astype(np.float32)
    q = np.rint(t.astype(np.float64)).astype(np.int8)
    s7 = (amax / np.float32(7.0)).astype(np.float32)
    return q.reshape(G, N, K), s7


def int4_dequant(q, s7) -> np.ndarray:
    """bf16(fl32(q * s7)): the bf16 weight value the bf16 matrix product consumes."""
    q = np.asarray(q, dtype=np.int8)
    G, N, K = q.shape
    prod = (q.reshape(G, N, K // 128, 128).astype(np.float32)
            * np.asarray(s7, np.float32)[:, :, :, None]).astype(np.float32)
    return bf16_round(prod).reshape(G, N, K)


def int4_dequant_exact(q, s7) -> np.ndarray:
    """q * s7 exactly (fp64): the weight value the 4-bit path on the FP8 matrix core
    stands for.  The codes -7..7 are exact e4m3 values and the product of a 3-bit integer
    and an fp32 scale is exact in fp64, so no rounding enters here."""
    q = np.asarray(q, dtype=np.int8)
    G, N, K = q.shape
    return (q.reshape(G, N, K // 128, 128).astype(np.float64)
            * np.asarray(s7, np.float32).astype(np.float64)[:, :, :, None]).reshape(G, N, K)


def int4_pack(q) -> np.ndarray:
    """Pack int4 codes [..., K] into bytes [..., K/2] (a storage layout of this library).

    Every 8 consecutive codes k = 8p .. 8p+7 fill the 4 bytes 4p .. 4p+3: byte 4p+b holds
    code 8p+b in its low nibble and code 8p+4+b in its high nibble.  A nibble is sign
    (bit 3, set for negative codes) and magnitude (bits 0-2); codes lie in [-7, 7].
    """
    q = np.asarray(q, dtype=np.int8)
    K = q.shape[-1]
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    if q.size and (q.min() < -7 or q.max() > 7):
        raise ValueError("int4 codes must lie in [-7, 7]")
    mag = np.abs(q.astype(np.int16))
    nib = np.where(q < 0, 8 | mag, mag).reshape(*q.shape[:-1], K // 8, 8)
    packed = nib[..., :4] | (nib[..., 4:] << 4)
    return packed.reshape(*q.shape[:-1], K // 2).astype(np.uint8)
