"""ctypes loader of ``libmoe_gfx950.so`` (the C ABI declared in include/moe.h).

Loading fails loudly when the library has not been built: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gfx950.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_HIP = -3
MOE_ERR_WORKSPACE = -4

MOE_F32, MOE_BF16, MOE_E4M3, MOE_INT4 = 0, 1, 2, 3
MOE_ROUTE_RENORM = 1
MOE_EPI_PLAIN, MOE_EPI_SWIGLU = 0, 1
MOE_MODE_FP32, MOE_MODE_FP8, MOE_MODE_W4A16, MOE_MODE_W4A8 = 0, 1, 2, 3
MOE_ROUTE_SCORE, MOE_ROUTE_HASH = 0, 1
MOE_LAYOUT_CONTIGUOUS, MOE_LAYOUT_MASKED = 0, 1

_P = C.c_void_p
_I = C.c_int
_U = C.c_uint
_D = C.c_double
_Z = C.c_size_t


class MoeLayerDesc(C.Structure):
    _fields_ = [("T", _I), ("d", _I), ("E", _I), ("k", _I), ("I", _I), ("mode", _I),
                ("route", _I), ("route_flags", _U), ("capacity_factor", _D), ("m_align", _I),
                ("layout", _I)]


class MoeLayerWeights(C.Structure):
    _fields_ = [("w_router", _P), ("bias", _P), ("w13", _P), ("s13", _P), ("w2", _P),
                ("s2", _P)]


# name -> (restype, argtypes); every symbol include/moe.h declares
SIGNATURES = {
    "moe_last_error": (C.c_char_p, []),
    "moe_device_supported": (_I, [_I]),
    "moe_capacity": (_I, [_I, _I, _I, _D]),
    "moe_rows_bound": (_Z, [_I, _I, _I, _I]),
    "moe_route": (_I, [_P, _I, _P, _P, _I, _I, _I, _I, _U, _P, _P, _P, _P, _Z, _P]),
    "moe_route_workspace_size": (_Z, [_I, _I, _I, _I]),
    "moe_route_noalloc": (_I, [_P, _I, _P, _P, _I, _I, _I, _I, _U, _P, _P, _P, _P]),
    "moe_route_from_logits": (_I, [_P, _P, _I, _I, _I, _U, _P, _P, _P]),
    "moe_route_hash": (_I, [_P, _I, _I, _P, _P, _P]),
    "moe_dispatch": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "moe_dispatch_masked": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_quant_fp8": (_I, [_P, _I, _I, _I, _P, _I, _I, _P, _P, _P]),
    "moe_quant_weight_fp8": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_pack_weight_fp8": (_I, [_P, _I, _I, _I, _P, _P]),
    "moe_quant_weight_int4": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "grouped_gemm_fp8": (_I, [_P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "grouped_gemm_fp8_masked": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "gemm_fp8": (_I, [_P, _P, _P, _P, _I, _I, _I, _P, _P]),
    "grouped_gemm_w4a16": (_I, [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "moe_pack_weight_int4": (_I, [_P, _P, _I, _I, _I, _P, _P, _P]),
    "grouped_gemm_w4a8": (_I, [_P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "grouped_gemm_f32": (_I, [_P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "moe_combine": (_I, [_P, _I, _P, _P, _I, _I, _I, _P, _I, _P]),
    "moe_layer_workspace_size": (_Z, [C.POINTER(MoeLayerDesc)]),
    "moe_layer_fwd": (_I, [C.POINTER(MoeLayerDesc), C.POINTER(MoeLayerWeights), _P, _P, _P, _P,
                           _Z, _P, _P]),
    "moe_probe_mfma_fp8": (_I, [_I, _I, C.c_uint8, _P, _P]),
    "moe_probe_hbm_read": (_I, [_P, _Z, _I, _P, _P]),
    "moe_layer_chunked_workspace_size": (_Z, [C.POINTER(MoeLayerDesc), _I]),
    "moe_layer_fwd_chunked": (_I, [C.POINTER(MoeLayerDesc), C.POINTER(MoeLayerWeights), _P, _P,
                                   _P, _P, _Z, _I, _P, _P]),
}

_lib = None


def load() -> C.CDLL:
    """Load the library once; raise ImportError if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m fp8_grouped_gemm_amd.build` (no CPU fallback exists)")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def check(status: int, fn: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, fn, load().moe_last_error().decode())
