"""Host-side checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments before touching a device.  No kernel runs here."""
import ctypes as C
import os
import re

import pytest

from fp8_grouped_gemm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = C.c_void_p(0x1000)   # never dereferenced: validation rejects the call first


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\*?\s*"
                       r"([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_symbols_exported():
    lib = _lib.load()
    declared = _declared()
    assert len(declared) == 29, declared
    for name in declared:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name
    assert sorted(_lib.SIGNATURES) == declared


def test_capacity_and_rows_bound(golden):
    lib = _lib.load()
    ex = golden["capacity_example"]
    assert lib.moe_capacity(ex["T"], ex["k"], ex["E"], ex["factor"]) == ex["value"]
    assert lib.moe_capacity(4096, 8, 256, 2.0) == 256
    assert lib.moe_capacity(100, 2, 7, 2.0) == 58   # ceil(200/7) = 29 -> 58
    assert lib.moe_capacity(10, 2, 4, 0.0) == 0
    assert lib.moe_capacity(-1, 2, 4, 1.0) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_rows_bound(4096, 8, 256, 128) == 4096 * 8 + 256 * 127
    assert lib.moe_rows_bound(4096, 8, 256, 0) == 0


def _err(status, fragment=None):
    lib = _lib.load()
    assert status == _lib.MOE_ERR_INVALID_ARG
    msg = lib.moe_last_error().decode()
    assert msg
    if fragment:
        assert fragment in msg, msg


def test_route_rejects_bad_args():
    lib = _lib.load()
    S = None
    _err(lib.moe_route_from_logits(None, None, 4, 8, 2, 0, FAKE, FAKE, S), "null")
    _err(lib.moe_route_from_logits(FAKE, None, 4, 8, 9, 0, FAKE, FAKE, S), "k must")
    _err(lib.moe_route_from_logits(FAKE, None, 4, 2000, 2, 0, FAKE, FAKE, S), "E must")
    _err(lib.moe_route_from_logits(FAKE, None, 4, 8, 2, 4, FAKE, FAKE, S), "flags")
    _err(lib.moe_route(FAKE, _lib.MOE_E4M3, FAKE, FAKE, 4, 256, 8, 2, 0, FAKE, FAKE, FAKE,
                       None, 0, S), "x_dt")
    _err(lib.moe_route(FAKE, _lib.MOE_BF16, FAKE, FAKE, 4, 200, 8, 2, 0, FAKE, FAKE, FAKE,
                       None, 0, S), "128")
    # split-K partial planes: T*E floats per plane, none for fp32 or tiny shapes
    n = lib.moe_route_workspace_size(128, 7168, 256, _lib.MOE_BF16)
    assert n > 0 and n % (128 * 256 * 4) == 0
    assert lib.moe_route_workspace_size(128, 7168, 256, _lib.MOE_F32) == 0
    _err(lib.moe_route_hash(None, 4, 8, FAKE, FAKE, S), "null")


def test_dispatch_and_quant_reject_bad_args():
    lib = _lib.load()
    S = None
    _err(lib.moe_dispatch(FAKE, 4, 2, 8, 0, 0, FAKE, FAKE, FAKE, FAKE, S), "m_align")
    _err(lib.moe_dispatch(FAKE, 4, 2, 8, 16, -1, FAKE, FAKE, FAKE, FAKE, S), "capacity")
    _err(lib.moe_dispatch(FAKE, 4, 2, 8, 16, 0, None, FAKE, FAKE, FAKE, S), "null")
    _err(lib.moe_quant_fp8(FAKE, _lib.MOE_BF16, 4, 100, None, 1, 4, FAKE, FAKE, S), "K must")
    _err(lib.moe_quant_fp8(FAKE, _lib.MOE_BF16, 4, 128, None, 1, 8, FAKE, FAKE, S), "rows_out")
    _err(lib.moe_quant_fp8(FAKE, _lib.MOE_INT4, 4, 128, None, 1, 4, FAKE, FAKE, S), "x_dt")
    _err(lib.moe_quant_weight_fp8(FAKE, 1, 100, 128, FAKE, FAKE, S), "multiples of 128")
    _err(lib.moe_pack_weight_fp8(FAKE, 1, 128, 200, C.c_void_p(0x2000), S), "multiples of 128")
    _err(lib.moe_pack_weight_fp8(FAKE, 1, 128, 128, FAKE, S), "overlap")
    _err(lib.moe_pack_weight_fp8(None, 1, 128, 128, FAKE, S), "null")
    _err(lib.gemm_fp8(FAKE, FAKE, FAKE, FAKE, 16, 128, 128 * 129, FAKE, S), "K must be <=")
    _err(lib.moe_quant_weight_int4(FAKE, 1, 8, 100, FAKE, FAKE, S), "K must")


def test_gemm_and_combine_reject_bad_args():
    lib = _lib.load()
    S = None
    _err(lib.grouped_gemm_fp8(FAKE, FAKE, None, 1, FAKE, FAKE, FAKE, 0, 128, 128, 128, 0,
                              _lib.MOE_BF16, FAKE, None, S), "G must")
    _err(lib.grouped_gemm_fp8(FAKE, FAKE, None, 1, FAKE, FAKE, FAKE, 2, 128, 100, 128, 0,
                              _lib.MOE_BF16, FAKE, None, S), "multiples of 128")
    _err(lib.grouped_gemm_fp8(FAKE, FAKE, None, 1, FAKE, FAKE, FAKE, 2, 128, 128, 128, 1,
                              _lib.MOE_BF16, FAKE, None, S), "SwiGLU")
    _err(lib.grouped_gemm_fp8(FAKE, FAKE, None, 1, FAKE, FAKE, FAKE, 2, 128, 128, 128, 7,
                              _lib.MOE_BF16, FAKE, None, S), "epilogue")
    _err(lib.grouped_gemm_fp8(FAKE, None, None, 1, FAKE, FAKE, FAKE, 2, 128, 128, 128, 0,
                              _lib.MOE_BF16, FAKE, None, S), "scale")
    _err(lib.grouped_gemm_fp8_masked(FAKE, FAKE, FAKE, FAKE, FAKE, 4, -1, 128, 128, 0,
                                     _lib.MOE_BF16, FAKE, None, S), "cap")
    _err(lib.grouped_gemm_fp8_masked(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 128, 100, 0,
                                     _lib.MOE_BF16, FAKE, None, S), "multiples of 128")
    _err(lib.gemm_fp8(FAKE, FAKE, FAKE, FAKE, 16, 384, 200, FAKE, S), "multiples of 128")
    # outputs overlapping the weight scales (read through the scalar cache)
    base = 0x100000
    _err(lib.gemm_fp8(FAKE, FAKE, FAKE, C.c_void_p(base), 16, 256, 256,
                      C.c_void_p(base + 8), S), "must not overlap sB")
    _err(lib.grouped_gemm_fp8(FAKE, FAKE, None, 1, FAKE, C.c_void_p(base), FAKE, 2, 64, 128, 256,
                              1, _lib.MOE_E4M3, FAKE, C.c_void_p(base + 16), S),
         "must not overlap sB")
    _err(lib.grouped_gemm_fp8_masked(FAKE, FAKE, FAKE, C.c_void_p(base), FAKE, 2, 16, 128, 128,
                                     0, _lib.MOE_BF16, C.c_void_p(base - 64), None, S),
         "must not overlap sB")
    _err(lib.gemm_fp8(None, FAKE, FAKE, FAKE, 16, 128, 128, FAKE, S), "null")
    _err(lib.grouped_gemm_w4a16(FAKE, None, 1, FAKE, FAKE, FAKE, 2, 64, 96, 128, 1, FAKE, S),
         "multiple of 128")
    _err(lib.grouped_gemm_f32(FAKE, None, 1, FAKE, FAKE, 2, 64, 24, 128, 0, FAKE, S),
         "multiple of 16")
    _err(lib.moe_combine(FAKE, _lib.MOE_BF16, FAKE, FAKE, 4, 2, 12, FAKE, _lib.MOE_BF16, S),
         "multiple of 8")
    _err(lib.moe_combine(FAKE, _lib.MOE_E4M3, FAKE, FAKE, 4, 2, 16, FAKE, _lib.MOE_BF16, S),
         "dtypes")


def test_layer_descriptor_checks_and_workspace():
    lib = _lib.load()
    D = _lib.MoeLayerDesc
    good = D(4096, 7168, 256, 8, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 0.0, 128)
    n = lib.moe_layer_workspace_size(C.byref(good))
    R = 4096 * 8 + 256 * 127
    # the big pieces: token codes, h codes, bf16 expert outputs
    assert n >= 4096 * 7168 + R * 2048 + R * 7168 * 2
    assert n < (4096 * 7168 + R * 2048 + R * 7168 * 2) * 1.05
    bad = D(4096, 7168, 256, 8, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_HASH, 0, 0.0, 128)
    assert lib.moe_layer_workspace_size(C.byref(bad)) == 0       # hash needs k = 1
    assert "hash" in lib.moe_last_error().decode()
    bad = D(16, 7168, 256, 8, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 0.0, 0)
    assert lib.moe_layer_workspace_size(C.byref(bad)) == 0
    w = _lib.MoeLayerWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    st = lib.moe_layer_fwd(C.byref(good), C.byref(w), FAKE, None, FAKE, FAKE, 16, None, None)
    assert st == _lib.MOE_ERR_WORKSPACE
    w = _lib.MoeLayerWeights(FAKE, None, FAKE, FAKE, FAKE, FAKE)
    st = lib.moe_layer_fwd(C.byref(good), C.byref(w), FAKE, None, FAKE, FAKE, n, None, None)
    assert st == _lib.MOE_ERR_INVALID_ARG
    # no tokens: x, y (and token_ids) may be null; with no counts to report nothing runs
    w = _lib.MoeLayerWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    empty = D(0, 7168, 256, 8, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 0.0, 128)
    n0 = lib.moe_layer_workspace_size(C.byref(empty))
    assert n0 > 0
    assert lib.moe_layer_fwd(C.byref(empty), C.byref(w), None, None, None, FAKE, n0, None,
                             None) == _lib.MOE_OK
    _err(lib.moe_layer_fwd(C.byref(good), C.byref(w), None, None, FAKE, FAKE, n, None, None),
         "null")


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_fp8_operands_beyond_32bit_offsets_rejected():
    """The FP8 GEMMs read activation rows with 32-bit byte offsets: operands whose rows
    reach past 2^32 - 256 bytes are rejected before any launch."""
    lib = _lib.load()
    S = None
    K = 16384
    rows = (1 << 32) // K                               # rows * K = 2^32
    _err(lib.gemm_fp8(FAKE, FAKE, FAKE, FAKE, rows, 128, K, FAKE, S), "32-bit")
    _err(lib.grouped_gemm_fp8(FAKE, FAKE, None, 1, FAKE, FAKE, FAKE, 2, rows, 128, K, 0,
                              _lib.MOE_BF16, FAKE, None, S), "32-bit")
    _err(lib.grouped_gemm_fp8_masked(FAKE, FAKE, FAKE, FAKE, FAKE, 4, rows // 4, 128, K, 0,
                                     _lib.MOE_BF16, FAKE, None, S), "32-bit")
    D = _lib.MoeLayerDesc
    # T * d = 600000 * 7168 > 2^32
    big_t = D(600000, 7168, 256, 8, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 0.0, 16)
    assert lib.moe_layer_workspace_size(C.byref(big_t)) == 0
    assert "32-bit" in lib.moe_last_error().decode()
    # rows * I: T * k * I > 2^32 with T * d below it
    big_r = D(300000, 7168, 256, 8, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 0.0, 16)
    assert lib.moe_layer_workspace_size(C.byref(big_r)) == 0
    assert "32-bit" in lib.moe_last_error().decode()
    # the same sizes without FP8 operands are accepted (bf16 / fp32 paths use 64-bit)
    ok = D(300000, 7168, 256, 8, 2048, _lib.MOE_MODE_W4A16, _lib.MOE_ROUTE_SCORE, 0, 0.0, 16)
    assert lib.moe_layer_workspace_size(C.byref(ok)) > 0


def test_masked_dispatch_and_layout_checks():
    lib = _lib.load()
    S = None
    _err(lib.moe_dispatch_masked(FAKE, 4, 2, 8, 0, FAKE, FAKE, FAKE, S), "capacity")
    _err(lib.moe_dispatch_masked(FAKE, 4, 2, 8, 4, None, FAKE, FAKE, S), "null")
    D = _lib.MoeLayerDesc
    # decode shape, capacity ceil(128*8/256) * 2 = 8: buffers of 256 * 8 rows
    m = D(128, 7168, 256, 8, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 2.0, 16,
          _lib.MOE_LAYOUT_MASKED)
    n = lib.moe_layer_workspace_size(C.byref(m))
    rows = 256 * 8
    assert n >= rows * 7168 + rows * 2048 + rows * 7168 * 2
    assert n < (rows * 7168 + rows * 2048 + rows * 7168 * 2) * 1.1
    no_cap = D(128, 7168, 256, 8, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 0.0, 16,
               _lib.MOE_LAYOUT_MASKED)
    assert lib.moe_layer_workspace_size(C.byref(no_cap)) == 0
    assert "capacity_factor" in lib.moe_last_error().decode()
    w4 = D(128, 7168, 256, 8, 2048, _lib.MOE_MODE_W4A16, _lib.MOE_ROUTE_SCORE, 0, 2.0, 16,
           _lib.MOE_LAYOUT_MASKED)
    assert lib.moe_layer_workspace_size(C.byref(w4)) == 0
    assert "MOE_MODE_FP8" in lib.moe_last_error().decode()
    bad = D(128, 7168, 256, 8, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 2.0, 16, 7)
    assert lib.moe_layer_workspace_size(C.byref(bad)) == 0
    assert "layout" in lib.moe_last_error().decode()
    # a positive factor whose capacity floors to 0 (ceil(4*2/256) * 0.5 = 0) is refused in
    # both layouts rather than read as dropless; with no tokens it is harmless
    for layout in (_lib.MOE_LAYOUT_CONTIGUOUS, _lib.MOE_LAYOUT_MASKED):
        tiny = D(4, 7168, 256, 2, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 0.5, 16,
                 layout)
        assert lib.moe_layer_workspace_size(C.byref(tiny)) == 0
        assert "capacity_factor" in lib.moe_last_error().decode()
        empty = D(0, 7168, 256, 2, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 0.5, 16,
                  layout)
        assert lib.moe_layer_workspace_size(C.byref(empty)) > 0


def test_chunked_pipeline_checks():
    lib = _lib.load()
    D = _lib.MoeLayerDesc
    d = D(4096, 7168, 256, 8, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 0.0, 16)
    one = D(256, 7168, 256, 8, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 0.0, 16)
    n = lib.moe_layer_chunked_workspace_size(C.byref(d), 256)
    # two regions, each a whole layer pass over 256 tokens
    assert n >= 2 * lib.moe_layer_workspace_size(C.byref(one))
    assert lib.moe_layer_chunked_workspace_size(C.byref(d), 0) == 0
    cap = D(4096, 7168, 256, 8, 2048, _lib.MOE_MODE_FP8, _lib.MOE_ROUTE_SCORE, 0, 1.0, 16)
    assert lib.moe_layer_chunked_workspace_size(C.byref(cap), 256) == 0
    w = _lib.MoeLayerWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    S = C.c_void_p(0x10)
    _err(lib.moe_layer_fwd_chunked(C.byref(d), C.byref(w), FAKE, None, FAKE, FAKE, n, 256, S, S),
         "stream_aux")
    _err(lib.moe_layer_fwd_chunked(C.byref(cap), C.byref(w), FAKE, None, FAKE, FAKE, n, 256, S,
                                   None), "dropless")
    _err(lib.moe_layer_fwd_chunked(C.byref(d), C.byref(w), FAKE, None, FAKE, FAKE, n, 0, S, None),
         "chunk_tokens")


def test_build_rejects_kernels_with_scratch():
    """The build's spill check reads the compiler's resource remarks: a kernel with private
    (scratch) memory is named, kernels without are not."""
    from fp8_grouped_gemm_amd.build import scratch_users
    remarks = """x.hip:1:1: remark: Function Name: _Zgood [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark: Function Name: _Zbad [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     ScratchSize [bytes/lane]: 44 [-Rpass-analysis=kernel-resource-usage]"""
    assert scratch_users(remarks) == ["_Zbad (44 bytes/lane)"]


def test_binding_runs_each_call_on_its_tensors_device():
    """Every binding call that takes tensors is wrapped so that it runs with the tensors'
    GPU current (the library launches on the current device); CPU tensors reach the
    call itself, which refuses them before anything is launched."""
    import torch
    import fp8_grouped_gemm_amd as M
    tensor_calls = [n for n in M.__all__ if n not in (
        "moe_device_supported", "moe_capacity", "moe_rows_bound", "moe_route_workspace_size",
        "moe_layer_workspace_size", "moe_layer_chunked_workspace_size", "MoeError", "LayerDesc",
        "moe_probe_mfma_fp8")]   # (takes a device, not tensors, and makes it current itself)
    for name in tensor_calls:
        assert hasattr(getattr(M, name), "__wrapped__"), name
    with pytest.raises(ValueError, match="on the GPU"):
        M.moe_combine(torch.zeros(4, 128), torch.zeros(4, dtype=torch.int32),
                      torch.zeros(4), 4, 1)


def test_probes_reject_bad_args():
    lib = _lib.load()
    S = None
    _err(lib.moe_probe_mfma_fp8(4, 10, 0x38, None, S), "null")
    _err(lib.moe_probe_mfma_fp8(0, 10, 0x38, FAKE, S), "n_blocks")
    _err(lib.moe_probe_mfma_fp8(4, 0, 0x38, FAKE, S), "iters")
    _err(lib.moe_probe_mfma_fp8(4, 10, 0x7F, FAKE, S), "NaN")
    _err(lib.moe_probe_mfma_fp8(4, 10, 0xFF, FAKE, S), "NaN")
    _err(lib.moe_probe_hbm_read(None, 1024, 4, FAKE, S), "null")
    _err(lib.moe_probe_hbm_read(FAKE, 1000, 4, FAKE, S), "multiple of 16")
    _err(lib.moe_probe_hbm_read(FAKE, 0, 4, FAKE, S), "multiple of 16")
    _err(lib.moe_probe_hbm_read(FAKE, 1024, 0, FAKE, S), "n_blocks")
