"""MI355X (gfx950) forward pass of one Mixture-of-Experts FFN layer.

A thin binding over the C ABI of ``libmoe_gfx950.so`` (include/moe.h): each function
here has the C entry point's name, takes torch tensors that live on the GPU, allocates
the outputs with torch and passes raw pointers plus the current HIP stream.  Every
step runs in the library's HIP kernels; nothing is computed in Python.
"""
from __future__ import annotations

import ctypes as C
import functools
from typing import Optional

import torch

from . import _lib
from ._lib import (MOE_BF16, MOE_E4M3, MOE_EPI_PLAIN, MOE_EPI_SWIGLU, MOE_F32, MOE_INT4,
                   MOE_MODE_FP32, MOE_MODE_FP8, MOE_MODE_W4A16, MOE_MODE_W4A8, MOE_ROUTE_HASH,
                   MOE_ROUTE_RENORM, MOE_ROUTE_SCORE, MoeError, MoeLayerDesc, MoeLayerWeights)

__all__ = [
    "moe_device_supported", "moe_capacity", "moe_rows_bound", "moe_route", "moe_route_noalloc",
    "moe_route_from_logits", "moe_route_hash", "moe_route_workspace_size", "moe_dispatch",
    "moe_dispatch_masked", "moe_quant_fp8",
    "moe_quant_weight_fp8", "moe_pack_weight_fp8", "moe_quant_weight_int4", "moe_pack_weight_int4",
    "grouped_gemm_fp8", "grouped_gemm_fp8_masked", "grouped_gemm_w4a8",
    "gemm_fp8", "grouped_gemm_w4a16",
    "grouped_gemm_f32", "moe_combine", "moe_layer_workspace_size", "moe_layer_fwd", "MoeError",
    "moe_layer_chunked_workspace_size", "moe_layer_fwd_chunked",
    "LayerDesc", "moe_probe_mfma_fp8", "moe_probe_hbm_read",
]


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _lib_():
    return _lib.load()


def _on_tensor_device(fn):
    """Run fn with the device of its GPU tensor arguments (and of the tensors in a dict
    argument, such as the layer's weights) current.  The library checks and launches on
    the current HIP device, and the stream passed in belongs to the tensors' device, so
    the two must agree; tensors on different GPUs are refused."""
    @functools.wraps(fn)
    def call(*args, **kwargs):
        flat = []
        for a in (*args, *kwargs.values()):
            flat.extend(a.values() if isinstance(a, dict) else (a,))
        devs = {a.device for a in flat if isinstance(a, torch.Tensor) and a.is_cuda}
        if len(devs) > 1:
            raise ValueError(f"{fn.__name__}: tensors on different devices {sorted(map(str, devs))}")
        if not devs:
            return fn(*args, **kwargs)
        with torch.cuda.device(devs.pop()):
            return fn(*args, **kwargs)
    return call


# --------------------------------------------------------------- host helpers

def moe_device_supported(device: int = 0) -> bool:
    return _lib_().moe_device_supported(device) == _lib.MOE_OK


def moe_capacity(T: int, k: int, E: int, factor: float) -> int:
    r = _lib_().moe_capacity(T, k, E, float(factor))
    _lib.check(min(r, 0), "moe_capacity")
    return r


def moe_rows_bound(T: int, k: int, E: int, m_align: int) -> int:
    return _lib_().moe_rows_bound(T, k, E, m_align)


# -------------------------------------------------------------------- routing

@_on_tensor_device
def moe_route(x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor, k: int,
              renorm: bool = False, use_workspace: bool = True):
    """Router logits + biased softmax top-k.  Returns (topk_idx, topk_w, logits).
    use_workspace=False passes no workspace (the logits GEMM then runs without split-K)."""
    T, d = x.shape
    E = w_router.shape[0]
    dev = x.device
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    nws = _lib_().moe_route_workspace_size(T, d, E, _dt(x)) if use_workspace else 0
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    _lib.check(_lib_().moe_route(_ptr(x), _dt(x), _ptr(w_router), _ptr(bias), T, d, E, k,
                                 MOE_ROUTE_RENORM if renorm else 0, _ptr(logits), _ptr(idx),
                                 _ptr(w), _ptr(ws), nws, _stream(dev)), "moe_route")
    return idx, w, logits


@_on_tensor_device
def moe_route_noalloc(x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor, k: int,
                      renorm: bool = False, out=None):
    """moe_route with the split-K partials in the library's static device scratch (no
    device allocation inside the call).  ``out`` = (topk_idx, topk_w, logits) tensors to
    write, or None to allocate them here with torch.  Returns (topk_idx, topk_w, logits)."""
    T, d = x.shape
    E = w_router.shape[0]
    dev = x.device
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((T, E), dtype=torch.float32, device=dev))
    idx, w, logits = out
    _lib.check(_lib_().moe_route_noalloc(_ptr(x), _dt(x), _ptr(w_router), _ptr(bias), T, d, E,
                                         k, MOE_ROUTE_RENORM if renorm else 0, _ptr(logits),
                                         _ptr(idx), _ptr(w), _stream(dev)), "moe_route_noalloc")
    return idx, w, logits


def moe_route_workspace_size(T: int, d: int, E: int, dtype=torch.bfloat16) -> int:
    return _lib_().moe_route_workspace_size(T, d, E, MOE_BF16 if dtype == torch.bfloat16 else MOE_F32)


@_on_tensor_device
def moe_route_from_logits(logits: torch.Tensor, bias: Optional[torch.Tensor], k: int,
                          renorm: bool = False):
    T, E = logits.shape
    dev = logits.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _lib.check(_lib_().moe_route_from_logits(_ptr(logits), _ptr(bias), T, E, k,
                                             MOE_ROUTE_RENORM if renorm else 0, _ptr(idx),
                                             _ptr(w), _stream(dev)), "moe_route_from_logits")
    return idx, w


@_on_tensor_device
def moe_route_hash(token_ids: torch.Tensor, E: int):
    T = token_ids.shape[0]
    dev = token_ids.device
    idx = torch.empty((T, 1), dtype=torch.int32, device=dev)
    w = torch.empty((T, 1), dtype=torch.float32, device=dev)
    _lib.check(_lib_().moe_route_hash(_ptr(token_ids), T, E, _ptr(idx), _ptr(w), _stream(dev)),
               "moe_route_hash")
    return idx, w


@_on_tensor_device
def moe_dispatch(topk_idx: torch.Tensor, E: int, m_align: int, capacity: int = 0):
    """Returns (counts [E], offsets [E+1], row_of_slot [T*k], slot_of_row [rows_bound])."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    R = moe_rows_bound(T, k, E, m_align)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ros = torch.empty(T * k, dtype=torch.int32, device=dev)
    sor = torch.empty(R, dtype=torch.int32, device=dev)
    _lib.check(_lib_().moe_dispatch(_ptr(topk_idx), T, k, E, m_align, capacity, _ptr(counts),
                                    _ptr(offsets), _ptr(ros), _ptr(sor), _stream(dev)),
               "moe_dispatch")
    return counts, offsets, ros, sor


@_on_tensor_device
def moe_dispatch_masked(topk_idx: torch.Tensor, E: int, capacity: int):
    """Fixed-capacity layout.  Returns (counts [E], row_of_slot [T*k], slot_of_row [E*C])."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    ros = torch.empty(T * k, dtype=torch.int32, device=dev)
    sor = torch.empty(E * capacity, dtype=torch.int32, device=dev)
    _lib.check(_lib_().moe_dispatch_masked(_ptr(topk_idx), T, k, E, capacity, _ptr(counts),
                                           _ptr(ros), _ptr(sor), _stream(dev)),
               "moe_dispatch_masked")
    return counts, ros, sor


# --------------------------------------------------------------- quantisation

@_on_tensor_device
def moe_quant_fp8(x: torch.Tensor, src_row: Optional[torch.Tensor] = None, src_div: int = 1,
                  rows_out: Optional[int] = None):
    """1x128 e4m3 quantisation; returns (codes uint8 [rows_out, K], scales fp32)."""
    rows_in, K = x.shape
    rows_out = rows_in if rows_out is None else rows_out
    dev = x.device
    q = torch.empty((rows_out, K), dtype=torch.uint8, device=dev)
    s = torch.empty((rows_out, K // 128), dtype=torch.float32, device=dev)
    _lib.check(_lib_().moe_quant_fp8(_ptr(x), _dt(x), rows_in, K, _ptr(src_row), src_div,
                                     rows_out, _ptr(q), _ptr(s), _stream(dev)), "moe_quant_fp8")
    return q, s


@_on_tensor_device
def moe_quant_weight_fp8(w: torch.Tensor):
    G, N, K = w.shape
    dev = w.device
    q = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
    s = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device=dev)
    _lib.check(_lib_().moe_quant_weight_fp8(_ptr(w), G, N, K, _ptr(q), _ptr(s), _stream(dev)),
               "moe_quant_weight_fp8")
    return q, s


@_on_tensor_device
def moe_pack_weight_fp8(q: torch.Tensor):
    """e4m3 codes [G, N, K] (or [N, K]) -> the fragment-major layout the FP8 GEMMs read
    (same shape and byte count; see moe_pack_weight_fp8 in include/moe.h)."""
    q3 = q if q.dim() == 3 else q[None]
    G, N, K = q3.shape
    q3 = q3.contiguous()                  # kept alive until the launch is enqueued
    out = torch.empty_like(q3)
    _lib.check(_lib_().moe_pack_weight_fp8(_ptr(q3), G, N, K, _ptr(out), _stream(q.device)),
               "moe_pack_weight_fp8")
    return out if q.dim() == 3 else out[0]


@_on_tensor_device
def moe_quant_weight_int4(w: torch.Tensor):
    G, N, K = w.shape
    dev = w.device
    q = torch.empty((G, N, K // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((G, N, K // 128), dtype=torch.float32, device=dev)
    _lib.check(_lib_().moe_quant_weight_int4(_ptr(w), G, N, K, _ptr(q), _ptr(s), _stream(dev)),
               "moe_quant_weight_int4")
    return q, s


@_on_tensor_device
def moe_pack_weight_int4(q: torch.Tensor, s7: torch.Tensor):
    """int4 codes [G, N, K/2] + scales [G, N, K/128] (moe_quant_weight_int4) -> the
    fragment-major order grouped_gemm_w4a8 reads (same shapes and byte counts)."""
    G, N, K2 = q.shape
    qf = torch.empty_like(q)
    s7f = torch.empty_like(s7)
    _lib.check(_lib_().moe_pack_weight_int4(_ptr(q), _ptr(s7), G, N, 2 * K2, _ptr(qf), _ptr(s7f),
                                            _stream(q.device)), "moe_pack_weight_int4")
    return qf, s7f


# --------------------------------------------------------------- grouped GEMM

@_on_tensor_device
def grouped_gemm_fp8(A, sA, B, sB, offsets, R_cap: int, N: int, swiglu: bool = False,
                     a_rows: Optional[torch.Tensor] = None, a_row_div: int = 1):
    """B: weight codes packed by moe_pack_weight_fp8.  Returns C bf16 [R_cap, N] (plain)
    or (codes e4m3 [R_cap, N], sC [R_cap, N/128])."""
    K = A.shape[1]
    G = B.shape[0]
    dev = A.device
    if swiglu:
        Cc = torch.empty((R_cap, N), dtype=torch.uint8, device=dev)
        sC = torch.empty((R_cap, N // 128), dtype=torch.float32, device=dev)
        out_dt, epi = MOE_E4M3, MOE_EPI_SWIGLU
    else:
        Cc = torch.empty((R_cap, N), dtype=torch.bfloat16, device=dev)
        sC = None
        out_dt, epi = MOE_BF16, MOE_EPI_PLAIN
    _lib.check(_lib_().grouped_gemm_fp8(_ptr(A), _ptr(sA), _ptr(a_rows), a_row_div, _ptr(B),
                                        _ptr(sB), _ptr(offsets), G, R_cap, N, K, epi, out_dt,
                                        _ptr(Cc), _ptr(sC), _stream(dev)), "grouped_gemm_fp8")
    return (Cc, sC) if swiglu else Cc


@_on_tensor_device
def grouped_gemm_w4a8(A, sA, B, s7, offsets, R_cap: int, N: int, swiglu: bool = False,
                      a_rows: Optional[torch.Tensor] = None, a_row_div: int = 1):
    """4-bit weights (packed by moe_pack_weight_int4) on the FP8 matrix core.  Returns C bf16
    [R_cap, N] (plain) or (codes e4m3 [R_cap, N], sC [R_cap, N/128])."""
    K = A.shape[1]
    G = B.shape[0]
    dev = A.device
    if swiglu:
        Cc = torch.empty((R_cap, N), dtype=torch.uint8, device=dev)
        sC = torch.empty((R_cap, N // 128), dtype=torch.float32, device=dev)
        out_dt, epi = MOE_E4M3, MOE_EPI_SWIGLU
    else:
        Cc = torch.empty((R_cap, N), dtype=torch.bfloat16, device=dev)
        sC = None
        out_dt, epi = MOE_BF16, MOE_EPI_PLAIN
    _lib.check(_lib_().grouped_gemm_w4a8(_ptr(A), _ptr(sA), _ptr(a_rows), a_row_div, _ptr(B),
                                         _ptr(s7), _ptr(offsets), G, R_cap, N, K, epi, out_dt,
                                         _ptr(Cc), _ptr(sC), _stream(dev)), "grouped_gemm_w4a8")
    return (Cc, sC) if swiglu else Cc


@_on_tensor_device
def grouped_gemm_fp8_masked(A, sA, B, sB, counts, cap: int, N: int, swiglu: bool = False):
    """Fixed-capacity layout: A [G*cap, K]; group g owns rows [g*cap, g*cap + counts[g]).
    Returns C bf16 [G*cap, N] (plain) or (codes e4m3 [G*cap, N], sC [G*cap, N/128])."""
    K = A.shape[1]
    G = B.shape[0]
    dev = A.device
    rows = G * cap
    if swiglu:
        Cc = torch.empty((rows, N), dtype=torch.uint8, device=dev)
        sC = torch.empty((rows, N // 128), dtype=torch.float32, device=dev)
        out_dt, epi = MOE_E4M3, MOE_EPI_SWIGLU
    else:
        Cc = torch.empty((rows, N), dtype=torch.bfloat16, device=dev)
        sC = None
        out_dt, epi = MOE_BF16, MOE_EPI_PLAIN
    _lib.check(_lib_().grouped_gemm_fp8_masked(_ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(counts),
                                               G, cap, N, K, epi, out_dt, _ptr(Cc), _ptr(sC),
                                               _stream(dev)), "grouped_gemm_fp8_masked")
    return (Cc, sC) if swiglu else Cc


@_on_tensor_device
def gemm_fp8(A, sA, B, sB):
    """Dense block-scaled FP8 GEMM: A [M, K] e4m3 + sA, B [N, K] e4m3 codes packed by
    moe_pack_weight_fp8 + sB -> bf16 [M, N]."""
    M, K = A.shape
    N = B.shape[0]
    Cc = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _lib.check(_lib_().gemm_fp8(_ptr(A), _ptr(sA), _ptr(B), _ptr(sB), M, N, K, _ptr(Cc),
                                _stream(A.device)), "gemm_fp8")
    return Cc


@_on_tensor_device
def grouped_gemm_w4a16(A, B, s7, offsets, R_cap: int, N: int, swiglu: bool = False,
                       a_rows: Optional[torch.Tensor] = None, a_row_div: int = 1):
    K = A.shape[1]
    G = B.shape[0]
    dev = A.device
    Cc = torch.empty((R_cap, N), dtype=torch.bfloat16, device=dev)
    _lib.check(_lib_().grouped_gemm_w4a16(_ptr(A), _ptr(a_rows), a_row_div, _ptr(B), _ptr(s7),
                                          _ptr(offsets), G, R_cap, N, K,
                                          MOE_EPI_SWIGLU if swiglu else MOE_EPI_PLAIN, _ptr(Cc),
                                          _stream(dev)), "grouped_gemm_w4a16")
    return Cc


@_on_tensor_device
def grouped_gemm_f32(A, B, offsets, R_cap: int, N: int, swiglu: bool = False,
                     a_rows: Optional[torch.Tensor] = None, a_row_div: int = 1):
    K = A.shape[1]
    G = B.shape[0]
    dev = A.device
    Cc = torch.empty((R_cap, N), dtype=torch.float32, device=dev)
    _lib.check(_lib_().grouped_gemm_f32(_ptr(A), _ptr(a_rows), a_row_div, _ptr(B), _ptr(offsets),
                                        G, R_cap, N, K,
                                        MOE_EPI_SWIGLU if swiglu else MOE_EPI_PLAIN, _ptr(Cc),
                                        _stream(dev)), "grouped_gemm_f32")
    return Cc


@_on_tensor_device
def moe_combine(o: torch.Tensor, row_of_slot: torch.Tensor, topk_w: torch.Tensor, T: int, k: int,
                out_dtype=torch.bfloat16):
    d = o.shape[1]
    dev = o.device
    y = torch.empty((T, d), dtype=out_dtype, device=dev)
    _lib.check(_lib_().moe_combine(_ptr(o), _dt(o), _ptr(row_of_slot), _ptr(topk_w), T, k, d,
                                   _ptr(y), _dt(y), _stream(dev)), "moe_combine")
    return y


# --------------------------------------------------------- measurement probes

def moe_probe_mfma_fp8(n_blocks: int, iters: int, code: int = 0x38,
                       device: Optional[torch.device] = None):
    """Enqueue the FP8 matrix-core probe on the current stream of `device` (default
    cuda:0); returns its fp32 output [n_blocks * 512] (n_blocks * 8 * iters * 4 * 65536
    FLOP are performed)."""
    dev = torch.device(device or "cuda:0")
    out = torch.empty(n_blocks * 512, dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _lib.check(_lib_().moe_probe_mfma_fp8(n_blocks, iters, code, _ptr(out), _stream(dev)),
                   "moe_probe_mfma_fp8")
    return out


@_on_tensor_device
def moe_probe_hbm_read(buf: torch.Tensor, n_blocks: int):
    """Enqueue the HBM read probe over the bytes of `buf`; returns the per-workgroup
    XORs of the 32-bit words read (uint32 stored as int32) [n_blocks]."""
    dev = buf.device
    out = torch.empty(n_blocks, dtype=torch.int32, device=dev)
    nbytes = buf.numel() * buf.element_size()
    _lib.check(_lib_().moe_probe_hbm_read(_ptr(buf), nbytes, n_blocks, _ptr(out), _stream(dev)),
               "moe_probe_hbm_read")
    return out


# ---------------------------------------------------------------------- layer

class LayerDesc:
    """Python view of moe_layer_desc."""

    def __init__(self, T, d, E, k, I, mode="fp8", route="score", renorm=False,
                 capacity_factor=0.0, m_align=128, layout="contiguous"):
        modes = {"fp32": MOE_MODE_FP32, "fp8": MOE_MODE_FP8, "w4a16": MOE_MODE_W4A16,
                 "w4a8": MOE_MODE_W4A8}
        layouts = {"contiguous": _lib.MOE_LAYOUT_CONTIGUOUS, "masked": _lib.MOE_LAYOUT_MASKED}
        self.c = MoeLayerDesc(T, d, E, k, I, modes[mode],
                              MOE_ROUTE_HASH if route == "hash" else MOE_ROUTE_SCORE,
                              MOE_ROUTE_RENORM if renorm else 0, float(capacity_factor), m_align,
                              layouts[layout])


def moe_layer_workspace_size(desc: LayerDesc) -> int:
    n = _lib_().moe_layer_workspace_size(C.byref(desc.c))
    if n == 0:
        raise MoeError(_lib.MOE_ERR_INVALID_ARG, "moe_layer_workspace_size",
                       _lib_().moe_last_error().decode())
    return n


@_on_tensor_device
def moe_layer_fwd(desc: LayerDesc, weights: dict, x: torch.Tensor,
                  token_ids: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  y: Optional[torch.Tensor] = None, counts: Optional[torch.Tensor] = None):
    """Whole layer forward.  ``weights`` holds w_router, bias, w13, s13, w2, s2 tensors
    (as moe_layer_weights).  Returns (y, counts)."""
    dev = x.device
    ws_bytes = moe_layer_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty(x.shape, dtype=x.dtype, device=dev)
    if counts is None:
        counts = torch.empty(desc.c.E, dtype=torch.int32, device=dev)
    w = MoeLayerWeights(*(_ptr(weights.get(n)) for n in ("w_router", "bias", "w13", "s13", "w2",
                                                        "s2")))
    _lib.check(_lib_().moe_layer_fwd(C.byref(desc.c), C.byref(w), _ptr(x), _ptr(token_ids),
                                     _ptr(y), _ptr(workspace), workspace.numel(), _ptr(counts),
                                     _stream(dev)), "moe_layer_fwd")
    return y, counts


def moe_layer_chunked_workspace_size(desc: LayerDesc, chunk_tokens: int) -> int:
    n = _lib_().moe_layer_chunked_workspace_size(C.byref(desc.c), chunk_tokens)
    if n == 0:
        raise MoeError(_lib.MOE_ERR_INVALID_ARG, "moe_layer_chunked_workspace_size",
                       _lib_().moe_last_error().decode() or "chunked pipeline not available "
                       "for this descriptor")
    return n


@_on_tensor_device
def moe_layer_fwd_chunked(desc: LayerDesc, weights: dict, x: torch.Tensor, chunk_tokens: int,
                          token_ids: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None,
                          y: Optional[torch.Tensor] = None,
                          aux_stream: Optional[torch.cuda.Stream] = None):
    """The layer forward as a two-stream chunk pipeline (chunk i's routing, dispatch and
    quantisation on ``aux_stream`` beside chunk i-1's GEMMs on the current stream).
    Returns y."""
    dev = x.device
    if workspace is None:
        workspace = torch.empty(moe_layer_chunked_workspace_size(desc, chunk_tokens),
                                dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty(x.shape, dtype=x.dtype, device=dev)
    if aux_stream is None:
        aux_stream = torch.cuda.Stream(device=dev)
    w = MoeLayerWeights(*(_ptr(weights.get(n)) for n in ("w_router", "bias", "w13", "s13", "w2",
                                                        "s2")))
    _lib.check(_lib_().moe_layer_fwd_chunked(C.byref(desc.c), C.byref(w), _ptr(x),
                                             _ptr(token_ids), _ptr(y), _ptr(workspace),
                                             workspace.numel(), chunk_tokens, _stream(dev),
                                             C.c_void_p(aux_stream.cuda_stream)),
               "moe_layer_fwd_chunked")
    return y
