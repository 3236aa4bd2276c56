"""Seeded synthetic inputs for the MoE FFN layer forward.

This module draws random numbers and nothing else: it holds none of the
layer's arithmetic (no quantisation, no routing, no GEMM).  Both the HIP path
and the CPU oracle consume what it returns, each applying the method's steps
itself.  Every tensor comes from its own ``torch.Generator`` seeded with
``(seed, tensor_id)``, so any tensor can be regenerated on its own.

Workload shapes follow the pages' DeepSeek-style MoE layers (see
``WORKLOADS``); value distributions are the ones the workloads state:
activations N(0, 1), weights N(0, std = 1/sqrt(fan_in)), router bias
U[-0.01, 0.01] (the small random bias initialisation recommended for the
aux-loss-free routing in the MegaMoE article, section 2.2).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np
import torch

# fixed tensor ids: one independent stream per tensor
_TID = {
    "x": 1, "w_gate_router": 2, "bias": 3, "w13": 4, "w2": 5, "token_ids": 6,
    "skew": 7, "gemm_a": 8, "gemm_b": 9, "group_sizes": 10, "logits": 11,
    "topk_idx": 12, "scale": 13,
}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and recipe of one MoE layer workload.

    mode: "fp32" (no quantisation), "fp8" (e4m3, 1x128 activation and
    128x128 weight block scales), "w4a16" (int4 1x128 per-channel weight
    blocks, bf16 activations), "w4a8" (the same int4 weights with 1x128 e4m3
    activations).
    """
    name: str
    T: int
    d: int
    E: int
    k: int
    I: int
    mode: str
    route: str = "score"          # "score" | "hash"
    skew_frac: float = 0.0        # fraction of experts whose bias gets +skew_add
    skew_add: float = 0.0
    m_align: int = 128
    vocab: int = 129280           # token-id range for hash routing
    seed: int = 0

    @property
    def R_cap(self) -> int:
        return self.T * self.k + self.E * (self.m_align - 1)


WORKLOADS = {
    # tiny fp32 layer: T=256, d=256, E=8, top-2, I=512
    "tiny_fp32": Workload("tiny_fp32", T=256, d=256, E=8, k=2, I=512, mode="fp32", m_align=16),
    # prefill layer at a DeepSeek-V3-like shape, 10% of experts skewed by +2.0
    "prefill_fp8": Workload("prefill_fp8", T=4096, d=7168, E=256, k=8, I=2048, mode="fp8",
                            skew_frac=0.1, skew_add=2.0, m_align=128),
    # decode layer: same experts, 128 tokens
    "decode_fp8": Workload("decode_fp8", T=128, d=7168, E=256, k=8, I=2048, mode="fp8",
                           m_align=16),
    # hash-routed layer with int4 expert weights
    "hash_w4a16": Workload("hash_w4a16", T=8192, d=4096, E=64, k=1, I=2048, mode="w4a16",
                           route="hash", m_align=128),
    # the same layer with the 4-bit weights on the FP8 matrix core (1x128 e4m3 activations)
    "hash_w4a8": Workload("hash_w4a8", T=8192, d=4096, E=64, k=1, I=2048, mode="w4a8",
                          route="hash", m_align=128),
}


def scaled(w: Workload, **kw) -> Workload:
    """A copy of ``w`` with some fields replaced (used for reduced-size cases)."""
    return dataclasses.replace(w, **kw)


def _gen(seed: int, tensor: str, device, extra: int = 0) -> torch.Generator:
    h = hashlib.sha256(f"{seed}/{_TID[tensor]}/{extra}".encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return g


def normal(shape, seed: int, tensor: str, device="cpu", std: float = 1.0, extra: int = 0,
           dtype=torch.float32) -> torch.Tensor:
    """N(0, std^2) samples in fp32 (optionally cast to ``dtype`` by torch)."""
    g = _gen(seed, tensor, device, extra)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t if dtype == torch.float32 else t.to(dtype)


def uniform(shape, lo: float, hi: float, seed: int, tensor: str, device="cpu",
            extra: int = 0) -> torch.Tensor:
    g = _gen(seed, tensor, device, extra)
    t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def layer_inputs(w: Workload, device="cpu", weights_device: Optional[str] = None,
                 seed: Optional[int] = None) -> dict:
    """Draw every input of one layer forward.

    Returns torch tensors:
      x      [T, d]    bf16 (fp32 for mode "fp32"), N(0,1) drawn in fp32 and cast by torch
      w_router [E, d]  router weight, N(0, 1/sqrt(d)); bf16 except mode "fp32"
      bias   [E]       fp32 U[-0.01, 0.01]; +skew_add on round(skew_frac*E) experts
      w13    [E, 2I, d] fp32 gate rows [0, I) then up rows [I, 2I), N(0, 1/sqrt(d))
      w2     [E, d, I] fp32 down projection, N(0, 1/sqrt(I))
      token_ids [T]    int64 U[0, vocab) (hash routing only)
    Expert weights are unquantised fp32: each side quantises them itself.
    """
    s = w.seed if seed is None else seed
    wdev = weights_device or device
    act_dtype = torch.float32 if w.mode == "fp32" else torch.bfloat16
    out = {}
    out["x"] = normal((w.T, w.d), s, "x", device, dtype=act_dtype)
    if w.route == "score":
        out["w_router"] = normal((w.E, w.d), s, "w_gate_router", device,
                                 std=1.0 / np.sqrt(w.d), dtype=act_dtype)
        b = uniform((w.E,), -0.01, 0.01, s, "bias", "cpu")
        if w.skew_frac > 0:
            n_skew = int(round(w.skew_frac * w.E))
            rng = np.random.default_rng([s, _TID["skew"]])
            chosen = rng.choice(w.E, n_skew, replace=False)
            b[torch.as_tensor(chosen)] += w.skew_add
        out["bias"] = b.to(device)
    else:
        g = _gen(s, "token_ids", device)
        out["token_ids"] = torch.randint(0, w.vocab, (w.T,), generator=g, device=device,
                                         dtype=torch.int64)
    out["w13"] = normal((w.E, 2 * w.I, w.d), s, "w13", wdev, std=1.0 / np.sqrt(w.d))
    out["w2"] = normal((w.E, w.d, w.I), s, "w2", wdev, std=1.0 / np.sqrt(w.I))
    return out


def expert_weights(w: Workload, which: str, device="cpu", seed: Optional[int] = None) -> torch.Tensor:
    """Only the w13 or w2 tensor of ``layer_inputs`` (same values)."""
    s = w.seed if seed is None else seed
    if which == "w13":
        return normal((w.E, 2 * w.I, w.d), s, "w13", device, std=1.0 / np.sqrt(w.d))
    return normal((w.E, w.d, w.I), s, "w2", device, std=1.0 / np.sqrt(w.I))


# ---------------------------------------------------------------- grouped GEMM

def zipf_group_sizes(total: int = 8192, groups: int = 16, s: float = 1.1, seed: int = 0):
    """Group sizes M_i ~ multinomial(total, p_i proportional to i^-s), i = 1..groups."""
    rng = np.random.default_rng(seed)
    p = np.arange(1, groups + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    return rng.multinomial(total, p).astype(np.int64)


def gemm_inputs(M_sizes, N: int, K: int, seed: int = 0, device="cpu", b_device=None) -> dict:
    """Standalone grouped GEMM operands before quantisation.

    a [sum(M), K] fp32 N(0,1) rows in group order; b [G, N, K] fp32 N(0,1).
    """
    M = int(np.sum(M_sizes))
    G = len(M_sizes)
    return {
        "a": normal((M, K), seed, "gemm_a", device),
        "b": normal((G, N, K), seed, "gemm_b", b_device or device),
        "group_sizes": np.asarray(M_sizes, dtype=np.int64),
    }


# ----------------------------------------------------------- routing operands

def random_logits(T: int, E: int, seed: int = 0, device="cpu", ties: bool = False) -> torch.Tensor:
    """fp32 router logits N(0,1); with ``ties`` values are snapped to a coarse grid so
    that exact ties between experts are common."""
    t = normal((T, E), seed, "logits", device)
    if ties:
        t = torch.round(t * 4) / 4
    return t


def random_topk(T: int, E: int, k: int, seed: int = 0, skew: float = 0.0) -> np.ndarray:
    """[T, k] int32 expert ids, distinct within a token; ``skew`` > 0 biases towards
    low expert ids (Zipf-like) to make unbalanced loads."""
    rng = np.random.default_rng([seed, _TID["topk_idx"]])
    if skew > 0:
        p = np.arange(1, E + 1, dtype=np.float64) ** (-skew)
        p /= p.sum()
    else:
        p = None
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        out[t] = rng.choice(E, k, replace=False, p=p)
    return out
