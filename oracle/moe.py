"""The MoE FFN layer forward, step by step, in fp64 numpy (oracle side).

Each function states the passage it follows.  Where the pages leave a step
open, the reading taken is stated in the docstring.
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import (bf16_round, dequant_fp8_act, dequant_fp8_weight, int4_dequant,
                     int4_dequant_exact, quant_fp8_act)


# --------------------------------------------------------------------- routing

def router_logits(x, w_router) -> np.ndarray:
    """Gate logits W_g x for every token, fp64 [T, E].

    The router is a single linear layer (discosf.com sec. 4.4; tqpw.cn sec. 2.3);
    x [T, d] and W_g [E, d] are taken at their stored precision and multiplied
    exactly enough in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float64)
    return x @ w.T


def topk_route(logits_f32, bias, k: int, renorm: bool = False):
    """Biased softmax top-k gate.

    s_i = softmax(W_g x + b_i) (discosf.com sec. 2.2), softmax taken in (at least)
    fp32 (tqpw.cn sec. 2.3).  Readings:
      * the selection key is fl32(logit + b) computed as one fp32 addition, and the
        same key feeds the softmax, so the bias moves both choice and weight;
      * experts are ordered by key, largest first; equal keys go to the lower index;
      * the weights are the full softmax over all E experts at the chosen indices
        (G(x)_i in y = sum_i G(x)_i E_i(x), discosf.com sec. 2.1); with ``renorm``
        they are divided by their sum, which equals softmax over the k selected keys
        (the top-k-then-softmax code of mooersco.com ch. 1; cf-1.com sec. 3.1 lists
        both choices).
    Returns idx int32 [T, k] and weights fp64 [T, k].
    """
    L = np.asarray(logits_f32, dtype=np.float32)
    b = np.asarray(bias, dtype=np.float32)
    if not np.all(np.isfinite(L)):
        raise ValueError("topk_route: logits must be finite")
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("topk_route: need 1 <= k <= E")
    key = (L + b[None, :]).astype(np.float32)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    experts = np.arange(E)
    for t in range(T):
        kt = key[t].astype(np.float64)
        order = np.lexsort((experts, -kt))      # primary: key desc; secondary: index asc
        sel = order[:k]
        z = np.exp(kt - kt.max())
        p = z / z.sum()
        idx[t] = sel
        w[t] = p[sel]
        if renorm:
            w[t] /= w[t].sum()
    return idx, w


def hash_route(token_ids, E: int):
    """Hash routing: expert = ((id * 2654435761) mod 2^32) mod E, weight 1, k = 1.

    hash(token_id) % num_experts (tqpw.cn sec. 2.2) with the multiplicative hash
    the workload fixes; evaluated in Python integers.
    """
    ids = [int(v) for v in np.asarray(token_ids).ravel()]
    idx = np.array([[((i * 2654435761) % (1 << 32)) % E] for i in ids], dtype=np.int32)
    return idx, np.ones((len(ids), 1), dtype=np.float64)


def capacity(T: int, k: int, E: int, factor: float) -> int:
    """Expert capacity floor(ceil(T*k/E) * factor); factor <= 0 means dropless (0).

    mooersco.com ch. 1 gives ceil(seq_len*k/N)*2 and sec. 2.5 gives
    int(k*tokens/E * 1.2) = 76 for k=2, 2048 tokens, 64 experts; this form
    reproduces both.
    """
    if factor <= 0:
        return 0
    return int(math.floor(math.ceil(T * k / E) * factor))


def rows_bound(T: int, k: int, E: int, m_align: int) -> int:
    """Rows an expert-contiguous buffer can need: T*k + E*(m_align-1)."""
    return T * k + E * (m_align - 1)


def dispatch(idx, E: int, m_align: int, cap: int = 0):
    """Expert grouping of routed slots (discosf.com sec. 2.1, 'concatenate the
    per-expert token sets'; group sizes as in sec. 3.2).

    Slot s = t*k + j carries token t to expert idx[t, j].  For every expert the
    slots keep their (token, slot) order (a stable order); with a capacity C > 0
    only the first C slots of each expert are kept and the rest are dropped
    silently (mooersco.com sec. 2.5).  Each expert's kept rows are padded up to a
    multiple of m_align.
    Returns counts [E] (slots routed, before capacity), offsets [E+1],
    row_of_slot [T*k] (-1 = dropped), slot_of_row [rows_bound] (-1 = padding).
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    flat = idx.ravel()
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("dispatch: expert id out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    kept = np.minimum(counts, cap) if cap > 0 else counts.copy()
    padded = ((kept + m_align - 1) // m_align) * m_align
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(padded)
    row_of_slot = np.full(T * k, -1, dtype=np.int32)
    slot_of_row = np.full(rows_bound(T, k, E, m_align), -1, dtype=np.int32)
    rank = np.zeros(E, dtype=np.int64)
    for s in range(T * k):                 # slots in (token, slot) order
        e = flat[s]
        r = rank[e]
        rank[e] += 1
        if cap > 0 and r >= cap:
            continue
        row = offsets[e] + r
        row_of_slot[s] = row
        slot_of_row[row] = s
    return counts, offsets, row_of_slot, slot_of_row


def dispatch_masked(idx, E: int, cap: int):
    """The fixed-capacity ("masked") expert layout, the second grouped layout of DeepGEMM's
    release notes (qidao123.com day 3), with the capacity rule of mooersco.com sec. 2.5:
    expert e owns the C = ``cap`` rows [e*C, e*C + C) whatever its load; its slots, in
    (token, slot) order, take rows e*C, e*C + 1, ... until the C rows are full, and the
    slots past them are dropped silently.
    Returns counts [E] (slots routed, before capacity), row_of_slot [T*k] (-1 = dropped)
    and slot_of_row [E*C] (-1 = row left empty).
    """
    if cap < 1:
        raise ValueError("dispatch_masked: capacity must be >= 1")
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    flat = idx.ravel()
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("dispatch_masked: expert id out of range")
    counts = np.zeros(E, dtype=np.int32)
    row_of_slot = np.full(T * k, -1, dtype=np.int32)
    slot_of_row = np.full(E * cap, -1, dtype=np.int32)
    for s in range(T * k):                 # slots in (token, slot) order
        e = flat[s]
        r = counts[e]
        counts[e] += 1
        if r < cap:
            row_of_slot[s] = e * cap + r
            slot_of_row[e * cap + r] = s
    return counts, row_of_slot, slot_of_row


# ----------------------------------------------------------------- expert math

def grouped_gemm(A, B, offsets) -> np.ndarray:
    """Grouped GEMM, one loop over groups: C[rows of g] = A[rows of g] @ B[g]^T.

    Groups differ in M and share N and K (discosf.com sec. 3.2; a loop of per-expert
    GEMMs is the plain form, cf-1.com sec. 4.2).  A [R, K], B [G, N, K] (the "nt"
    operand layout), fp64.  Rows outside [0, offsets[G]) are zero.
    """
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    G = B.shape[0]
    C = np.zeros((A.shape[0], B.shape[1]), dtype=np.float64)
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            C[lo:hi] = A[lo:hi] @ B[g].T
    return C


def grouped_gemm_w4a8(qA, sA, q, s7, offsets) -> np.ndarray:
    """Grouped GEMM of 1x128 e4m3 activations with block-wise 4-bit weights: C[r, n] = sum
    over K blocks kb of sA[r,kb] * s7[g,n,kb] * sum_{k in kb} e4m3(qA[r,k]) * q[g,n,k]
    (the lecture's 4-bit weights, tqpw.cn sec. 3.1, promoted per 128-deep block as the
    FP8 path, qidao123.com day 3) -- the product of the dequantised operands, in fp64."""
    return grouped_gemm(dequant_fp8_act(qA, sA), int4_dequant_exact(q, s7), offsets)


def grouped_gemm_fp8(qA, sA, qB, sB, offsets) -> np.ndarray:
    """FP8 grouped GEMM with fine-grained scales, evaluated exactly enough.

    C[r, n] = sum over K blocks kb of sA[r,kb] * sB[g, n/128, kb] * sum_{k in kb}
    e4m3(qA[r,k]) * e4m3(qB[g,n,k]) -- the blockwise-promoted product (qidao123.com
    day 3, two-level accumulation) equals the product of the dequantised operands,
    which is what is computed here in fp64.
    """
    return grouped_gemm(dequant_fp8_act(qA, sA), dequant_fp8_weight(qB, sB), offsets)


def silu(z):
    """silu(z) = z / (1 + exp(-z)) in fp64 (numerically safe form for large |z|)."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def swiglu(g, u):
    """SwiGLU gate: silu(gate) * up.  The pages name the SwiGLU FFN (tqpw.cn sec.
    3.1, mooersco.com ch. 1) without a formula; this is the standard form
    (parity unpinned beyond its textbook special cases)."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def combine(o, row_of_slot, w, T: int, k: int) -> np.ndarray:
    """y_t = sum_j w[t,j] * o[row_of_slot[t*k+j]] in fp64, j in order, dropped
    slots skipped (y = sum_{i in TopK} G(x)_i E_i(x), discosf.com sec. 2.1)."""
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64).reshape(T, k)
    ros = np.asarray(row_of_slot, dtype=np.int64).reshape(T, k)
    y = np.zeros((T, o.shape[1]), dtype=np.float64)
    for j in range(k):
        r = ros[:, j]
        keep = r >= 0
        y[keep] += w[keep, j:j + 1] * o[r[keep]]
    return y


# ------------------------------------------------------------------ the layer

def layer_forward(mode: str, x, *, E: int, k: int, I: int, m_align: int = 16,
                  w_router=None, bias=None, token_ids=None, renorm: bool = False,
                  cap_factor: float = 0.0, experts=None, tokens=None, keep: bool = False):
    """One MoE FFN layer forward on one GPU's batch, fp64.

    mode "fp32":  w13 [E,2I,d], w2 [E,d,I] fp32 arrays in ``experts``; no quantisation.
    mode "fp8":   experts = (q13, s13, q2, s2), e4m3 codes with 128x128 scales; x is
                  quantised per token 1x128 (dynamic activation quantisation,
                  discosf.com sec. 4.2); h = swiglu(...) is rounded to fp32 and
                  requantised 1x128 before the down projection.
    mode "w4a16": experts = (c13, s13, c2, s2) int4 codes with 1x128 per-channel
                  scales; x is used as bf16 directly; h is rounded to fp32 then bf16.
    mode "w4a8":  the same int4 codes and scales, the weights taken exactly as q * s7
                  (the codes are exact e4m3 operands); x and h quantised 1x128 e4m3 as in
                  mode "fp8".
    Routing: score (softmax + bias top-k) when ``w_router`` is given, else hash.
    ``tokens`` (optional) restricts the expert computation to those tokens (every
    routing decision is still made for the whole batch); y rows of other tokens
    are NaN.  ``keep`` also returns, per computed slot, the activation row, the exact
    g, u and h = swiglu(g, u) before requantisation, and the dequantised weights of
    every expert used (for error analysis in tests).
    Returns a dict with logits32, idx, w, dispatch outputs, o rows and y (fp64).
    """
    x = np.asarray(x)
    T, d = x.shape
    xf = x.astype(np.float32)
    out = {}
    if w_router is not None:
        logits = router_logits(xf, w_router)
        L32 = logits.astype(np.float32)
        out["logits"] = logits
        idx, w = topk_route(L32, bias, k, renorm)
    else:
        idx, w = hash_route(token_ids, E)
    out["idx"], out["w"] = idx, w
    cap = capacity(T, k, E, cap_factor)
    counts, offsets, ros, sor = dispatch(idx, E, m_align, cap)
    out.update(counts=counts, offsets=offsets, row_of_slot=ros, slot_of_row=sor)

    want = np.ones(T, dtype=bool) if tokens is None else np.isin(np.arange(T), tokens)
    if mode in ("fp8", "w4a8"):
        qx, sx = quant_fp8_act(xf)
        xin = dequant_fp8_act(qx, sx)
        out["qx"], out["sx"] = qx, sx
    else:
        xin = xf.astype(np.float64)

    o, info, deq = {}, {}, {}
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        slots = sor[rows]
        slots = slots[slots >= 0]
        toks = slots // k
        sel = want[toks]
        slots, toks = slots[sel], toks[sel]
        if len(toks) == 0:
            continue
        a = xin[toks]
        if mode == "fp32":
            w13, w2 = np.asarray(experts[0][e], np.float64), np.asarray(experts[1][e], np.float64)
        elif mode == "fp8":
            q13, s13, q2, s2 = experts
            w13 = dequant_fp8_weight(q13[e:e + 1], s13[e:e + 1])[0]
            w2 = dequant_fp8_weight(q2[e:e + 1], s2[e:e + 1])[0]
        elif mode == "w4a8":
            c13, s13, c2, s2 = experts
            w13 = int4_dequant_exact(c13[e:e + 1], s13[e:e + 1])[0]
            w2 = int4_dequant_exact(c2[e:e + 1], s2[e:e + 1])[0]
        else:
            c13, s13, c2, s2 = experts
            w13 = int4_dequant(c13[e:e + 1], s13[e:e + 1])[0].astype(np.float64)
            w2 = int4_dequant(c2[e:e + 1], s2[e:e + 1])[0].astype(np.float64)
        gu = a @ w13.T
        h = swiglu(gu[:, :I], gu[:, I:])
        h_exact = h
        if mode in ("fp8", "w4a8"):
            qh, sh = quant_fp8_act(h.astype(np.float32))
            h = dequant_fp8_act(qh, sh)
        elif mode == "w4a16":
            h = bf16_round(h.astype(np.float32)).astype(np.float64)
        oe = h @ w2.T
        for i, s in enumerate(slots):
            o[int(s)] = oe[i]
            if keep:
                info[int(s)] = {"e": e, "a": a[i], "g": gu[i, :I], "u": gu[i, I:],
                                "h": h_exact[i], "h_used": h[i]}
        if keep:
            deq[e] = (w13, w2)
    y = np.full((T, d), np.nan, dtype=np.float64)
    wk = np.asarray(w).reshape(T, k)
    for t in np.nonzero(want)[0]:
        acc = np.zeros(d, dtype=np.float64)
        for j in range(k):
            s = t * k + j
            if ros[s] >= 0:
                acc += wk[t, j] * o[s]
        y[t] = acc
    out["o_by_slot"] = o
    out["y"] = y
    if keep:
        out["slot_info"], out["experts_deq"] = info, deq
    return out
