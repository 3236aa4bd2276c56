// C ABI of the MoE layer library: argument checks, device checks, workspace layout
// and the kernel sequence of the layer forward.  Declarations and contracts are in
// include/moe.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/moe.h"
#include "launch.hpp"
#include "tiles.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

#define REQUIRE(cond, ...) \
  do {                     \
    if (!(cond)) return fail(MOE_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];    // 0 unknown, 1 gfx950, -1 other
std::atomic<int> g_dev_cus[kMaxDevices];

int check_device(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d out of range", dev);
  int st = g_dev_ok[dev].load();
  if (st == 0) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(MOE_ERR_UNSUPPORTED, "hipGetDeviceProperties(%d): %s", dev, hipGetErrorString(e));
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_dev_cus[dev].store(prop.multiProcessorCount);
    g_dev_ok[dev].store(st);
  }
  if (st < 0) return fail(MOE_ERR_UNSUPPORTED, "device %d is not gfx950: FP8 kernels need MI355X", dev);
  return MOE_OK;
}

// current device must be gfx950; fills the CU count
int current_device(int* cus) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_UNSUPPORTED, "no HIP device: %s", hipGetErrorString(e));
  int st = check_device(dev);
  if (st != MOE_OK) return st;
  if (cus) *cus = g_dev_cus[dev].load();
  return MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

// Rows per small-group GEMM tile from the average rows per group: decode-sized groups
// use 16-row tiles, everything else 32-row tiles (measured best at the prefill shape,
// where most groups hold about 20 rows); groups above it use 128-row tiles.
int pick_bm(double avg_rows, bool swiglu) {
  (void)swiglu;
  return avg_rows <= 16 ? 16 : 32;
}

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// ------------------------------------------------------------ pure validation
int v_route_from_logits(const void* logits, int T, int E, int k, unsigned flags, const void* idx,
                        const void* w) {
  REQUIRE(logits && idx && w, "moe_route_from_logits: null pointer");
  REQUIRE(T >= 0, "T must be >= 0 (got %d)", T);
  REQUIRE(E >= 1 && E <= 1024, "E must be in [1, 1024] (got %d)", E);
  REQUIRE(k >= 1 && k <= E && k <= 64, "k must be in [1, min(E, 64)] (got %d)", k);
  REQUIRE((flags & ~MOE_ROUTE_RENORM) == 0, "unknown route flags 0x%x", flags);
  return MOE_OK;
}

int v_dispatch(const void* idx, int T, int k, int E, int m_align, int cap, const void* counts,
               const void* offsets, const void* ros, const void* sor) {
  REQUIRE(counts && offsets && sor, "moe_dispatch: null pointer");
  REQUIRE((idx && ros) || T == 0, "moe_dispatch: null pointer");
  REQUIRE(T >= 0 && k >= 1 && E >= 1 && E <= 65536, "moe_dispatch: bad T/k/E (%d/%d/%d)", T, k, E);
  REQUIRE(m_align >= 1 && m_align <= 1024, "m_align must be in [1, 1024] (got %d)", m_align);
  REQUIRE(cap >= 0, "capacity must be >= 0 (got %d)", cap);
  REQUIRE((long long)T * k + (long long)E * (m_align - 1) < (1LL << 31), "rows bound overflows int32");
  return MOE_OK;
}

// true if the byte ranges [a, a + na) and [b, b + nb) share a byte
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return a && b && na && nb && x < y + nb && y < x + na;
}

// The FP8 GEMM reads the weight scales through the scalar cache, which a store of the
// same launch would not update: its outputs must not overlap them.
int v_fp8_out_vs_scales(const char* fn, const float* sB, int G, int Nb, int K, const void* C,
                        const float* sC, long long rows, int N, bool swiglu) {
  const size_t nsb = (size_t)G * (Nb / 128) * (K / 128) * sizeof(float);
  const size_t nc = (size_t)rows * N * (swiglu ? 1 : 2);
  const size_t nsc = swiglu ? (size_t)rows * (N / 128) * sizeof(float) : 0;
  REQUIRE(!overlaps(sB, nsb, C, nc) && !overlaps(sB, nsb, sC, nsc),
          "%s: C and sC must not overlap sB", fn);
  return MOE_OK;
}

int v_gemm_common(const void* A, const void* B, const void* offsets, int G, int R_cap, int N,
                  int K, int epilogue, const void* C) {
  REQUIRE(A && B && offsets && C, "grouped GEMM: null pointer");
  REQUIRE(G >= 1 && G <= 1024, "G must be in [1, 1024] (got %d)", G);
  REQUIRE(R_cap >= 0, "R_cap must be >= 0");
  REQUIRE(N >= 1 && K >= 1, "N and K must be positive");
  REQUIRE(epilogue == MOE_EPI_PLAIN || epilogue == MOE_EPI_SWIGLU, "unknown epilogue %d", epilogue);
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

int moe_device_supported(int hip_device) { return check_device(hip_device); }

int moe_capacity(int T, int k, int E, double factor) {
  REQUIRE(T >= 0 && k >= 1 && E >= 1, "moe_capacity: bad T/k/E");
  REQUIRE(std::isfinite(factor), "moe_capacity: factor must be finite");
  if (factor <= 0) return 0;
  const long long tk = (long long)T * k;
  const long long c = (tk + E - 1) / E;
  const double v = std::floor((double)c * factor);
  REQUIRE(v < 2147483647.0, "moe_capacity: overflow");
  return (int)v;
}

size_t moe_rows_bound(int T, int k, int E, int m_align) {
  if (T < 0 || k < 1 || E < 1 || m_align < 1) return 0;
  return (size_t)T * k + (size_t)E * (m_align - 1);
}

int moe_route_from_logits(const float* logits, const float* bias, int T, int E, int k,
                          unsigned flags, int32_t* topk_idx, float* topk_w, void* stream) {
  int st = v_route_from_logits(logits, T, E, k, flags, topk_idx, topk_w);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if ((st = current_device(nullptr))) return st;
  // with one partial plane the kernel only reads the logits
  return hip_status(moe::launch_topk(const_cast<float*>(logits), nullptr, 1, bias, T, E, k,
                                     flags & MOE_ROUTE_RENORM, topk_idx, topk_w, S(stream)),
                    "topk launch");
}

size_t moe_route_workspace_size(int T, int d, int E, moe_dtype x_dt) {
  if (T <= 0 || E < 1 || d < 128 || x_dt != MOE_BF16 || d % 128) return 0;
  const int n = moe::router_splits(T, d, E, true);
  return n > 1 ? (size_t)n * T * E * sizeof(float) : 0;
}

int moe_route(const void* x, moe_dtype x_dt, const void* w_router, const float* bias, int T, int d,
              int E, int k, unsigned flags, float* logits, int32_t* topk_idx, float* topk_w,
              void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(x && w_router, "moe_route: null pointer");
  REQUIRE(x_dt == MOE_BF16 || x_dt == MOE_F32, "moe_route: x_dt must be MOE_BF16 or MOE_F32");
  REQUIRE(d >= 1, "moe_route: d must be positive");
  REQUIRE(x_dt != MOE_BF16 || d % 128 == 0, "moe_route: bf16 needs d %% 128 == 0 (got %d)", d);
  int st = v_route_from_logits(logits, T, E, k, flags, topk_idx, topk_w);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if ((st = current_device(nullptr))) return st;
  const size_t need = moe_route_workspace_size(T, d, E, x_dt);
  const int n_part = (need > 0 && ws && ws_bytes >= need)
                         ? moe::router_splits(T, d, E, x_dt == MOE_BF16) : 1;
  float* part = static_cast<float*>(ws);
  if ((st = hip_status(moe::launch_router(x, x_dt == MOE_BF16, w_router, logits, T, d, E, part,
                                          n_part, S(stream)),
                       "router launch")))
    return st;
  return hip_status(moe::launch_topk(logits, part, n_part, bias, T, E, k,
                                     flags & MOE_ROUTE_RENORM, topk_idx, topk_w, S(stream)),
                    "topk launch");
}

int moe_route_hash(const int64_t* token_ids, int T, int E, int32_t* topk_idx, float* topk_w,
                   void* stream) {
  REQUIRE(token_ids && topk_idx && topk_w, "moe_route_hash: null pointer");
  REQUIRE(T >= 0 && E >= 1, "moe_route_hash: bad T/E");
  if (T == 0) return MOE_OK;
  int st = current_device(nullptr);
  if (st) return st;
  return hip_status(moe::launch_hash_route(token_ids, T, E, topk_idx, topk_w, S(stream)),
                    "hash route launch");
}

int moe_dispatch(const int32_t* topk_idx, int T, int k, int E, int m_align, int capacity,
                 int32_t* counts, int32_t* offsets, int32_t* row_of_slot, int32_t* slot_of_row,
                 void* stream) {
  int st = v_dispatch(topk_idx, T, k, E, m_align, capacity, counts, offsets, row_of_slot,
                      slot_of_row);
  if (st) return st;
  if ((st = current_device(nullptr))) return st;
  const int rb = (int)moe_rows_bound(T, k, E, m_align);
  return hip_status(moe::launch_dispatch(topk_idx, T, k, E, m_align, capacity, counts, offsets,
                                         row_of_slot, slot_of_row, rb, S(stream)),
                    "dispatch launch");
}

int moe_quant_fp8(const void* x, moe_dtype x_dt, int rows_in, int K, const int32_t* src_row,
                  int src_div, int rows_out, uint8_t* q, float* scales, void* stream) {
  REQUIRE(x && q && scales, "moe_quant_fp8: null pointer");
  REQUIRE(x_dt == MOE_BF16 || x_dt == MOE_F32, "moe_quant_fp8: x_dt must be MOE_BF16 or MOE_F32");
  REQUIRE(K >= 128 && K % 128 == 0, "moe_quant_fp8: K must be a positive multiple of 128 (got %d)", K);
  REQUIRE(rows_in >= 0 && rows_out >= 0, "moe_quant_fp8: negative row count");
  REQUIRE(src_div >= 1, "moe_quant_fp8: src_div must be >= 1");
  REQUIRE(src_row || rows_out <= rows_in, "moe_quant_fp8: rows_out > rows_in without src_row");
  if (rows_out == 0) return MOE_OK;
  int st = current_device(nullptr);
  if (st) return st;
  return hip_status(moe::launch_quant_act(x, x_dt == MOE_BF16, K, src_row, src_div, rows_out, q,
                                          scales, S(stream)),
                    "quant launch");
}

int moe_quant_weight_fp8(const float* w, int G, int N, int K, uint8_t* q, float* scales,
                         void* stream) {
  REQUIRE(w && q && scales, "moe_quant_weight_fp8: null pointer");
  REQUIRE(G >= 1 && G <= 65535, "moe_quant_weight_fp8: G must be in [1, 65535]");
  REQUIRE(N >= 128 && N % 128 == 0 && K >= 128 && K % 128 == 0,
          "moe_quant_weight_fp8: N and K must be positive multiples of 128 (got %d, %d)", N, K);
  int st = current_device(nullptr);
  if (st) return st;
  return hip_status(moe::launch_quant_weight_fp8(w, G, N, K, q, scales, S(stream)),
                    "weight quant launch");
}

int moe_pack_weight_fp8(const uint8_t* q, int G, int N, int K, uint8_t* qf, void* stream) {
  REQUIRE(q && qf, "moe_pack_weight_fp8: null pointer");
  REQUIRE(q != qf, "moe_pack_weight_fp8: q and qf must not overlap");
  REQUIRE(G >= 1 && G <= 65535, "moe_pack_weight_fp8: G must be in [1, 65535]");
  REQUIRE(N > 0 && K > 0 && N % 128 == 0 && K % 128 == 0,
          "moe_pack_weight_fp8: N and K must be positive multiples of 128 (got %d, %d)", N, K);
  int st = current_device(nullptr);
  if (st) return st;
  return hip_status(moe::launch_pack_weight_fp8(q, G, N, K, qf, S(stream)), "fp8 pack launch");
}

int moe_quant_weight_int4(const float* w, int G, int N, int K, uint8_t* q, float* s7,
                          void* stream) {
  REQUIRE(w && q && s7, "moe_quant_weight_int4: null pointer");
  REQUIRE(G >= 1 && N >= 1, "moe_quant_weight_int4: bad G/N");
  REQUIRE(K >= 128 && K % 128 == 0, "moe_quant_weight_int4: K must be a positive multiple of 128");
  int st = current_device(nullptr);
  if (st) return st;
  return hip_status(moe::launch_quant_weight_int4(w, G, N, K, q, s7, S(stream)),
                    "int4 quant launch");
}

int grouped_gemm_fp8(const uint8_t* A, const float* sA, const int32_t* a_rows, int a_row_div,
                     const uint8_t* B, const float* sB, const int32_t* offsets, int G, int R_cap,
                     int N, int K, int epilogue, moe_dtype out_dt, void* C, float* sC,
                     void* stream) {
  int st = v_gemm_common(A, B, offsets, G, R_cap, N, K, epilogue, C);
  if (st) return st;
  REQUIRE(sA && sB, "grouped_gemm_fp8: null scale pointer");
  REQUIRE(N % 128 == 0 && K % 128 == 0, "grouped_gemm_fp8: N and K must be multiples of 128");
  REQUIRE(K / 128 <= moe::kGemmMaxKBlocks, "grouped_gemm_fp8: K must be <= %d",
          128 * moe::kGemmMaxKBlocks);
  REQUIRE(a_row_div >= 1, "grouped_gemm_fp8: a_row_div must be >= 1");
  const bool swiglu = epilogue == MOE_EPI_SWIGLU;
  if (swiglu) {
    REQUIRE(out_dt == MOE_E4M3 && sC, "grouped_gemm_fp8: SwiGLU epilogue writes e4m3 + sC");
  } else {
    REQUIRE(out_dt == MOE_BF16, "grouped_gemm_fp8: plain epilogue writes bf16");
  }
  if ((st = v_fp8_out_vs_scales("grouped_gemm_fp8", sB, G, swiglu ? 2 * N : N, K, C, sC, R_cap,
                                N, swiglu)))
    return st;
  if (R_cap == 0) return MOE_OK;
  int cus = 0;
  if ((st = current_device(&cus))) return st;
  const int bm = pick_bm((double)R_cap / G, swiglu);
  return hip_status(moe::launch_gemm_fp8(A, sA, a_rows, a_row_div, B, sB, offsets, G, R_cap, N, K,
                                         swiglu, C, sC, bm, cus, S(stream)),
                    "grouped_gemm_fp8 launch");
}

int grouped_gemm_fp8_masked(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB,
                            const int32_t* counts, int G, int cap, int N, int K, int epilogue,
                            moe_dtype out_dt, void* C, float* sC, void* stream) {
  REQUIRE(cap >= 0, "grouped_gemm_fp8_masked: cap must be >= 0");
  REQUIRE((long long)G * cap < (1LL << 31), "grouped_gemm_fp8_masked: G * cap overflows int32");
  const int rows = G * cap;
  int st = v_gemm_common(A, B, counts, G, rows, N, K, epilogue, C);
  if (st) return st;
  REQUIRE(sA && sB, "grouped_gemm_fp8_masked: null scale pointer");
  REQUIRE(N % 128 == 0 && K % 128 == 0,
          "grouped_gemm_fp8_masked: N and K must be multiples of 128");
  REQUIRE(K / 128 <= moe::kGemmMaxKBlocks, "grouped_gemm_fp8_masked: K must be <= %d",
          128 * moe::kGemmMaxKBlocks);
  const bool swiglu = epilogue == MOE_EPI_SWIGLU;
  if (swiglu) {
    REQUIRE(out_dt == MOE_E4M3 && sC, "grouped_gemm_fp8_masked: SwiGLU epilogue writes e4m3 + sC");
  } else {
    REQUIRE(out_dt == MOE_BF16, "grouped_gemm_fp8_masked: plain epilogue writes bf16");
  }
  if ((st = v_fp8_out_vs_scales("grouped_gemm_fp8_masked", sB, G, swiglu ? 2 * N : N, K, C, sC,
                                rows, N, swiglu)))
    return st;
  if (rows == 0) return MOE_OK;
  int cus = 0;
  if ((st = current_device(&cus))) return st;
  return hip_status(moe::launch_gemm_fp8(A, sA, nullptr, 1, B, sB, counts, G, rows, N, K, swiglu,
                                         C, sC, pick_bm(cap, swiglu), cus, S(stream),
                                         moe::kRowsMasked, cap),
                    "grouped_gemm_fp8_masked launch");
}

int gemm_fp8(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB, int M, int N,
             int K, uint16_t* C, void* stream) {
  REQUIRE(B && sB && (M == 0 || (A && sA && C)), "gemm_fp8: null pointer");
  REQUIRE(M >= 0 && N >= 128 && K >= 128, "gemm_fp8: bad sizes");
  REQUIRE(N % 128 == 0 && K % 128 == 0, "gemm_fp8: N and K must be multiples of 128");
  REQUIRE(K / 128 <= moe::kGemmMaxKBlocks, "gemm_fp8: K must be <= %d",
          128 * moe::kGemmMaxKBlocks);
  int st = v_fp8_out_vs_scales("gemm_fp8", sB, 1, N, K, C, nullptr, M, N, false);
  if (st) return st;
  if (M == 0) return MOE_OK;
  int cus = 0;
  st = current_device(&cus);
  if (st) return st;
  return hip_status(moe::launch_gemm_fp8(A, sA, nullptr, 1, B, sB, nullptr, 1, M, N, K, false, C,
                                         nullptr, pick_bm(M, false), cus, S(stream),
                                         moe::kRowsDense, M),
                    "gemm_fp8 launch");
}

int grouped_gemm_w4a16(const uint16_t* A, const int32_t* a_rows, int a_row_div, const uint8_t* B,
                       const float* s7, const int32_t* offsets, int G, int R_cap, int N, int K,
                       int epilogue, uint16_t* C, void* stream) {
  int st = v_gemm_common(A, B, offsets, G, R_cap, N, K, epilogue, C);
  if (st) return st;
  REQUIRE(s7, "grouped_gemm_w4a16: null scale pointer");
  REQUIRE(K % 128 == 0, "grouped_gemm_w4a16: K must be a multiple of 128");
  REQUIRE(N % 128 == 0, "grouped_gemm_w4a16: N must be a multiple of 128");
  REQUIRE(a_row_div >= 1, "grouped_gemm_w4a16: a_row_div must be >= 1");
  if (R_cap == 0) return MOE_OK;
  int cus = 0;
  if ((st = current_device(&cus))) return st;
  return hip_status(moe::launch_gemm_w4a16(A, a_rows, a_row_div, B, s7, offsets, G, R_cap, N, K,
                                           epilogue == MOE_EPI_SWIGLU, C, cus, S(stream)),
                    "grouped_gemm_w4a16 launch");
}

int grouped_gemm_f32(const float* A, const int32_t* a_rows, int a_row_div, const float* B,
                     const int32_t* offsets, int G, int R_cap, int N, int K, int epilogue,
                     float* C, void* stream) {
  int st = v_gemm_common(A, B, offsets, G, R_cap, N, K, epilogue, C);
  if (st) return st;
  REQUIRE(N % 16 == 0, "grouped_gemm_f32: N must be a multiple of 16");
  REQUIRE(a_row_div >= 1, "grouped_gemm_f32: a_row_div must be >= 1");
  if (R_cap == 0) return MOE_OK;
  if ((st = current_device(nullptr))) return st;
  return hip_status(moe::launch_gemm_f32(A, a_rows, a_row_div, B, offsets, G, R_cap, N, K,
                                         epilogue == MOE_EPI_SWIGLU, C, S(stream)),
                    "grouped_gemm_f32 launch");
}

int moe_combine(const void* o, moe_dtype o_dt, const int32_t* row_of_slot, const float* topk_w,
                int T, int k, int d, void* y, moe_dtype y_dt, void* stream) {
  REQUIRE(o && row_of_slot && topk_w && y, "moe_combine: null pointer");
  REQUIRE((o_dt == MOE_BF16 || o_dt == MOE_F32) && (y_dt == MOE_BF16 || y_dt == MOE_F32),
          "moe_combine: dtypes must be MOE_BF16 or MOE_F32");
  REQUIRE(T >= 0 && k >= 1, "moe_combine: bad T/k");
  REQUIRE(d >= 8 && d % 8 == 0, "moe_combine: d must be a positive multiple of 8");
  if (T == 0) return MOE_OK;
  int st = current_device(nullptr);
  if (st) return st;
  return hip_status(moe::launch_combine(o, o_dt == MOE_BF16, row_of_slot, topk_w, T, k, d, y,
                                        y_dt == MOE_BF16, S(stream)),
                    "combine launch");
}

// ------------------------------------------------------------------- layer
namespace {

struct LayerWs {
  size_t part, logits, idx, w, counts, offsets, ros, sor, qx, sx, h, sh, o, total;
};

int layer_check(const moe_layer_desc* d) {
  REQUIRE(d, "moe_layer: null descriptor");
  REQUIRE(d->T >= 0 && d->d >= 128 && d->E >= 1 && d->E <= 1024 && d->k >= 1 && d->I >= 1,
          "moe_layer: bad sizes T=%d d=%d E=%d k=%d I=%d", d->T, d->d, d->E, d->k, d->I);
  REQUIRE(d->k <= d->E && d->k <= 64, "moe_layer: k must be <= min(E, 64)");
  REQUIRE(d->mode == MOE_MODE_FP32 || d->mode == MOE_MODE_FP8 || d->mode == MOE_MODE_W4A16,
          "moe_layer: unknown mode %d", d->mode);
  REQUIRE(d->route == MOE_ROUTE_SCORE || d->route == MOE_ROUTE_HASH, "moe_layer: unknown route %d",
          d->route);
  REQUIRE(d->route != MOE_ROUTE_HASH || d->k == 1, "moe_layer: hash routing needs k = 1");
  REQUIRE((d->route_flags & ~MOE_ROUTE_RENORM) == 0, "moe_layer: unknown route flags");
  REQUIRE(std::isfinite(d->capacity_factor), "moe_layer: capacity_factor must be finite");
  REQUIRE(d->m_align >= 1 && d->m_align <= 1024, "moe_layer: m_align must be in [1, 1024]");
  REQUIRE(d->d % 128 == 0, "moe_layer: d must be a multiple of 128");
  if (d->mode == MOE_MODE_FP8) {
    REQUIRE(d->I % 128 == 0, "moe_layer: fp8 needs I %% 128 == 0");
    REQUIRE(d->d <= 128 * moe::kGemmMaxKBlocks && d->I <= 128 * moe::kGemmMaxKBlocks,
            "moe_layer: fp8 needs d, I <= %d", 128 * moe::kGemmMaxKBlocks);
  }
  if (d->mode == MOE_MODE_W4A16) REQUIRE(d->I % 128 == 0, "moe_layer: w4a16 needs I %% 128 == 0");
  if (d->mode == MOE_MODE_FP32) REQUIRE(d->I % 16 == 0, "moe_layer: fp32 needs I %% 16 == 0");
  REQUIRE((long long)d->T * d->k + (long long)d->E * (d->m_align - 1) < (1LL << 31),
          "moe_layer: rows bound overflows int32");
  return MOE_OK;
}

LayerWs layer_ws(const moe_layer_desc* d) {
  LayerWs L{};
  const size_t T = d->T, E = d->E, k = d->k, D = d->d, I = d->I;
  const size_t R = moe_rows_bound(d->T, d->k, d->E, d->m_align);
  size_t p = 0;
  auto take = [&](size_t bytes) { size_t at = p; p = align_up(p + bytes); return at; };
  L.part = take(d->route == MOE_ROUTE_SCORE && d->mode != MOE_MODE_FP32
                    ? moe_route_workspace_size(d->T, d->d, d->E, MOE_BF16) : 0);
  L.logits = take(d->route == MOE_ROUTE_SCORE ? T * E * 4 : 0);
  L.idx = take(T * k * 4);
  L.w = take(T * k * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.ros = take(T * k * 4);
  L.sor = take(R * 4);
  if (d->mode == MOE_MODE_FP8) {
    L.qx = take(T * D);
    L.sx = take(T * (D / 128) * 4);
    L.h = take(R * I);
    L.sh = take(R * (I / 128) * 4);
    L.o = take(R * D * 2);
  } else if (d->mode == MOE_MODE_W4A16) {
    L.h = take(R * I * 2);
    L.o = take(R * D * 2);
  } else {
    L.h = take(R * I * 4);
    L.o = take(R * D * 4);
  }
  L.total = p;
  return L;
}

}  // namespace

size_t moe_layer_workspace_size(const moe_layer_desc* desc) {
  if (layer_check(desc) != MOE_OK) return 0;
  return layer_ws(desc).total;
}

int moe_layer_fwd(const moe_layer_desc* d, const moe_layer_weights* w, const void* x,
                  const int64_t* token_ids, void* y, void* ws, size_t ws_bytes, int32_t* counts_out,
                  void* stream) {
  int st = layer_check(d);
  if (st) return st;
  REQUIRE(w && x && y && ws, "moe_layer_fwd: null pointer");
  REQUIRE(w->w13 && w->w2, "moe_layer_fwd: null expert weights");
  if (d->mode != MOE_MODE_FP32) REQUIRE(w->s13 && w->s2, "moe_layer_fwd: null weight scales");
  if (d->route == MOE_ROUTE_SCORE)
    REQUIRE(w->w_router && w->bias, "moe_layer_fwd: score routing needs w_router and bias");
  else
    REQUIRE(token_ids, "moe_layer_fwd: hash routing needs token_ids");
  const LayerWs L = layer_ws(d);
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "moe_layer_fwd: workspace %zu < %zu bytes", ws_bytes, L.total);
  if (d->T == 0) return MOE_OK;
  int cus = 0;
  if ((st = current_device(&cus))) return st;

  const hipStream_t s = S(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* logits = reinterpret_cast<float*>(base + L.logits);
  int32_t* idx = reinterpret_cast<int32_t*>(base + L.idx);
  float* gw = reinterpret_cast<float*>(base + L.w);
  int32_t* counts = counts_out ? counts_out : reinterpret_cast<int32_t*>(base + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* ros = reinterpret_cast<int32_t*>(base + L.ros);
  int32_t* sor = reinterpret_cast<int32_t*>(base + L.sor);
  const int T = d->T, D = d->d, E = d->E, k = d->k, I = d->I;
  const int R = (int)moe_rows_bound(T, k, E, d->m_align);
  const bool f32 = d->mode == MOE_MODE_FP32;

#define STEP(expr, what) \
  if ((st = hip_status((expr), what))) return st;

  if (d->route == MOE_ROUTE_SCORE) {
    const int n_part = f32 ? 1 : moe::router_splits(T, D, E, true);
    float* part = reinterpret_cast<float*>(base + L.part);
    STEP(moe::launch_router(x, !f32, w->w_router, logits, T, D, E, part, n_part, s),
         "router launch");
    STEP(moe::launch_topk(logits, part, n_part, w->bias, T, E, k,
                          d->route_flags & MOE_ROUTE_RENORM, idx, gw, s),
         "topk launch");
  } else {
    STEP(moe::launch_hash_route(token_ids, T, E, idx, gw, s), "hash route launch");
  }
  const int cap = moe_capacity(T, k, E, d->capacity_factor);
  if (cap < 0) return cap;
  STEP(moe::launch_dispatch(idx, T, k, E, d->m_align, cap, counts, offsets, ros, sor, R, s),
       "dispatch launch");
  const double avg = (double)T * k / E;
  void* o = base + L.o;
  if (d->mode == MOE_MODE_FP8) {
    uint8_t* qx = base + L.qx;
    float* sx = reinterpret_cast<float*>(base + L.sx);
    uint8_t* hq = base + L.h;
    float* sh = reinterpret_cast<float*>(base + L.sh);
    STEP(moe::launch_quant_act(x, true, D, nullptr, 1, T, qx, sx, s), "quant launch");
    STEP(moe::launch_gemm_fp8(qx, sx, sor, k, static_cast<const uint8_t*>(w->w13), w->s13, offsets,
                              E, R, I, D, true, hq, sh, pick_bm(avg, true), cus, s),
         "gemm1 launch");
    STEP(moe::launch_gemm_fp8(hq, sh, nullptr, 1, static_cast<const uint8_t*>(w->w2), w->s2,
                              offsets, E, R, D, I, false, o, nullptr, pick_bm(avg, false), cus, s),
         "gemm2 launch");
  } else if (d->mode == MOE_MODE_W4A16) {
    uint16_t* h = reinterpret_cast<uint16_t*>(base + L.h);
    STEP(moe::launch_gemm_w4a16(static_cast<const uint16_t*>(x), sor, k,
                                static_cast<const uint8_t*>(w->w13), w->s13, offsets, E, R, I, D,
                                true, h, cus, s),
         "gemm1 launch");
    STEP(moe::launch_gemm_w4a16(h, nullptr, 1, static_cast<const uint8_t*>(w->w2), w->s2, offsets,
                                E, R, D, I, false, static_cast<uint16_t*>(o), cus, s),
         "gemm2 launch");
  } else {
    float* h = reinterpret_cast<float*>(base + L.h);
    STEP(moe::launch_gemm_f32(static_cast<const float*>(x), sor, k,
                              static_cast<const float*>(w->w13), offsets, E, R, I, D, true, h, s),
         "gemm1 launch");
    STEP(moe::launch_gemm_f32(h, nullptr, 1, static_cast<const float*>(w->w2), offsets, E, R, D, I,
                              false, static_cast<float*>(o), s),
         "gemm2 launch");
  }
  STEP(moe::launch_combine(o, !f32, ros, gw, T, k, D, y, !f32, s), "combine launch");
#undef STEP
  return MOE_OK;
}

}  // extern "C"
