// C ABI of the MoE layer library: argument checks, device checks, workspace layout
// and the kernel sequence of the layer forward.  Declarations and contracts are in
// include/moe.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
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

// Rows per small-group GEMM tile from the rows an entry point is given per group
// (R_cap / G, which includes each group's padding up to m_align - 1 rows): decode-sized
// groups (at most 32 rows per group, i.e. about 16 live rows at m_align = 16) use
// 16-row tiles, everything else 32-row tiles (measured best at the prefill shape, where
// most groups hold about 20 rows); groups above the small-tile size use 128-row tiles.
// The layer applies the same rule to its own rows bound, so the layer and the entry
// point pick the same kernel for the same problem.
int pick_bm(double rows_per_group) { return rows_per_group <= 32 ? 16 : 32; }

// 256 x 256 tiles (a second kernel, launched first) for the whole 256-row tiles of the
// groups that hold them, where the groups average at least 256 rows and K spans an even
// number of 128-deep blocks.  Opt-in: FP8GG_BIG_TILES=1 in the environment (read at each
// call) turns them on; measured on MI355X they are still slower than the 128-row tiles
// alone (dense 8192 x 4096 x 7168: 1.79 vs 1.96 PFLOP/s).  The result meets the same error
// bound either way (bit-identical in the measured cases).
bool want_big(double rows_per_group, int K) {
  const char* e = std::getenv("FP8GG_BIG_TILES");
  if (!e || e[0] != '1') return false;
  return rows_per_group >= 256 && (K / 128) % 2 == 0;
}

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// The FP8 GEMM addresses its activation operand through a buffer resource with 32-bit
// byte offsets (row * K): every row it reads must end below this bound.
constexpr long long kMaxOperandBytes = (1LL << 32) - 256;

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

int moe_route_noalloc(const void* x, moe_dtype x_dt, const void* w_router, const float* bias,
                      int T, int d, int E, int k, unsigned flags, float* logits,
                      int32_t* topk_idx, float* topk_w, void* stream) {
  REQUIRE(x && w_router, "moe_route_noalloc: null pointer");
  REQUIRE(x_dt == MOE_BF16 || x_dt == MOE_F32,
          "moe_route_noalloc: x_dt must be MOE_BF16 or MOE_F32");
  REQUIRE(d >= 1, "moe_route_noalloc: d must be positive");
  REQUIRE(x_dt != MOE_BF16 || d % 128 == 0, "moe_route_noalloc: bf16 needs d %% 128 == 0 (got %d)",
          d);
  int st = v_route_from_logits(logits, T, E, k, flags, topk_idx, topk_w);
  if (st) return st;
  const size_t need = moe_route_workspace_size(T, d, E, x_dt);
  REQUIRE(need <= moe::kRouteScratchBytes,
          "moe_route_noalloc: %zu bytes of partial logits exceed the static scratch of %zu bytes "
          "(T * E too large; use moe_route with a workspace)",
          need, moe::kRouteScratchBytes);
  if (T == 0) return MOE_OK;
  if ((st = current_device(nullptr))) return st;
  const int n_part = need > 0 ? moe::router_splits(T, d, E, x_dt == MOE_BF16) : 1;
  void* part = nullptr;
  if (n_part > 1 && (st = hip_status(moe::route_scratch(&part), "router scratch address")))
    return st;
  if ((st = hip_status(moe::launch_router(x, x_dt == MOE_BF16, w_router, logits, T, d, E,
                                          static_cast<float*>(part), n_part, S(stream)),
                       "router launch")))
    return st;
  return hip_status(moe::launch_topk(logits, static_cast<float*>(part), n_part, bias, T, E, k,
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

int moe_dispatch_masked(const int32_t* topk_idx, int T, int k, int E, int capacity,
                        int32_t* counts, int32_t* row_of_slot, int32_t* slot_of_row,
                        void* stream) {
  REQUIRE(counts && slot_of_row, "moe_dispatch_masked: null pointer");
  REQUIRE((topk_idx && row_of_slot) || T == 0, "moe_dispatch_masked: null pointer");
  REQUIRE(T >= 0 && k >= 1 && E >= 1 && E <= 65536, "moe_dispatch_masked: bad T/k/E (%d/%d/%d)",
          T, k, E);
  REQUIRE(capacity >= 1, "moe_dispatch_masked: capacity must be >= 1 (got %d)", capacity);
  REQUIRE((long long)E * capacity < (1LL << 31) && (long long)T * k < (1LL << 31),
          "moe_dispatch_masked: E * capacity overflows int32");
  int st = current_device(nullptr);
  if (st) return st;
  return hip_status(moe::launch_dispatch(topk_idx, T, k, E, 1, capacity, counts, nullptr,
                                         row_of_slot, slot_of_row, E * capacity, S(stream), true),
                    "masked dispatch launch");
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
  REQUIRE(a_rows || (long long)R_cap * K <= kMaxOperandBytes,
          "grouped_gemm_fp8: R_cap * K = %lld exceeds the 32-bit operand offset range",
          (long long)R_cap * K);
  if ((st = v_fp8_out_vs_scales("grouped_gemm_fp8", sB, G, swiglu ? 2 * N : N, K, C, sC, R_cap,
                                N, swiglu)))
    return st;
  if (R_cap == 0) return MOE_OK;
  int cus = 0;
  if ((st = current_device(&cus))) return st;
  const int bm = pick_bm((double)R_cap / G);
  return hip_status(moe::launch_gemm_fp8(A, sA, a_rows, a_row_div, B, sB, offsets, G, R_cap, N, K,
                                         swiglu, C, sC, bm, cus, S(stream), moe::kRowsOffsets, 0,
                                         want_big((double)R_cap / G, K)),
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
  REQUIRE((long long)rows * K <= kMaxOperandBytes,
          "grouped_gemm_fp8_masked: G * cap * K = %lld exceeds the 32-bit operand offset range",
          (long long)rows * K);
  if ((st = v_fp8_out_vs_scales("grouped_gemm_fp8_masked", sB, G, swiglu ? 2 * N : N, K, C, sC,
                                rows, N, swiglu)))
    return st;
  if (rows == 0) return MOE_OK;
  int cus = 0;
  if ((st = current_device(&cus))) return st;
  return hip_status(moe::launch_gemm_fp8(A, sA, nullptr, 1, B, sB, counts, G, rows, N, K, swiglu,
                                         C, sC, pick_bm(cap), cus, S(stream),
                                         moe::kRowsMasked, cap, want_big(cap, K)),
                    "grouped_gemm_fp8_masked launch");
}

int moe_pack_weight_int4(const uint8_t* q, const float* s7, int G, int N, int K, uint8_t* qf,
                         float* s7f, void* stream) {
  REQUIRE(q && s7 && qf && s7f, "moe_pack_weight_int4: null pointer");
  REQUIRE(q != qf && (const void*)s7 != (const void*)s7f,
          "moe_pack_weight_int4: outputs must not overlap inputs");
  REQUIRE(G >= 1 && G <= 65535, "moe_pack_weight_int4: G must be in [1, 65535]");
  REQUIRE(N > 0 && K > 0 && N % 128 == 0 && K % 128 == 0,
          "moe_pack_weight_int4: N and K must be positive multiples of 128 (got %d, %d)", N, K);
  int st = current_device(nullptr);
  if (st) return st;
  return hip_status(moe::launch_pack_weight_int4(q, s7, G, N, K, qf, s7f, S(stream)),
                    "int4 pack launch");
}

int grouped_gemm_w4a8(const uint8_t* A, const float* sA, const int32_t* a_rows, int a_row_div,
                      const uint8_t* B, const float* s7, const int32_t* offsets, int G, int R_cap,
                      int N, int K, int epilogue, moe_dtype out_dt, void* C, float* sC,
                      void* stream) {
  int st = v_gemm_common(A, B, offsets, G, R_cap, N, K, epilogue, C);
  if (st) return st;
  REQUIRE(sA && s7, "grouped_gemm_w4a8: null scale pointer");
  REQUIRE(N % 128 == 0 && K % 128 == 0, "grouped_gemm_w4a8: N and K must be multiples of 128");
  REQUIRE(K / 128 <= moe::kGemmMaxKBlocks, "grouped_gemm_w4a8: K must be <= %d",
          128 * moe::kGemmMaxKBlocks);
  REQUIRE(a_row_div >= 1, "grouped_gemm_w4a8: a_row_div must be >= 1");
  const bool swiglu = epilogue == MOE_EPI_SWIGLU;
  if (swiglu) {
    REQUIRE(out_dt == MOE_E4M3 && sC, "grouped_gemm_w4a8: SwiGLU epilogue writes e4m3 + sC");
  } else {
    REQUIRE(out_dt == MOE_BF16, "grouped_gemm_w4a8: plain epilogue writes bf16");
  }
  REQUIRE(a_rows || (long long)R_cap * K <= kMaxOperandBytes,
          "grouped_gemm_w4a8: R_cap * K = %lld exceeds the 32-bit operand offset range",
          (long long)R_cap * K);
  if (R_cap == 0) return MOE_OK;
  int cus = 0;
  if ((st = current_device(&cus))) return st;
  return hip_status(moe::launch_gemm_w4a8(A, sA, a_rows, a_row_div, B, s7, offsets, G, R_cap, N,
                                          K, swiglu, C, sC, pick_bm((double)R_cap / G), cus,
                                          S(stream)),
                    "grouped_gemm_w4a8 launch");
}

int gemm_fp8(const uint8_t* A, const float* sA, const uint8_t* B, const float* sB, int M, int N,
             int K, uint16_t* C, void* stream) {
  REQUIRE(B && sB && (M == 0 || (A && sA && C)), "gemm_fp8: null pointer");
  REQUIRE(M >= 0 && N >= 128 && K >= 128, "gemm_fp8: bad sizes");
  REQUIRE(N % 128 == 0 && K % 128 == 0, "gemm_fp8: N and K must be multiples of 128");
  REQUIRE(K / 128 <= moe::kGemmMaxKBlocks, "gemm_fp8: K must be <= %d",
          128 * moe::kGemmMaxKBlocks);
  REQUIRE((long long)M * K <= kMaxOperandBytes,
          "gemm_fp8: M * K = %lld exceeds the 32-bit operand offset range", (long long)M * K);
  int st = v_fp8_out_vs_scales("gemm_fp8", sB, 1, N, K, C, nullptr, M, N, false);
  if (st) return st;
  if (M == 0) return MOE_OK;
  int cus = 0;
  st = current_device(&cus);
  if (st) return st;
  return hip_status(moe::launch_gemm_fp8(A, sA, nullptr, 1, B, sB, nullptr, 1, M, N, K, false, C,
                                         nullptr, pick_bm(M), cus, S(stream),
                                         moe::kRowsDense, M, want_big(M, K)),
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

// ------------------------------------------------------------ measurement probes
int moe_probe_mfma_fp8(int n_blocks, int iters, uint8_t code, float* out, void* stream) {
  REQUIRE(out, "moe_probe_mfma_fp8: null pointer");
  REQUIRE(n_blocks >= 1 && n_blocks <= 65536, "moe_probe_mfma_fp8: n_blocks must be in [1, 65536]");
  REQUIRE(iters >= 1, "moe_probe_mfma_fp8: iters must be positive");
  REQUIRE((code & 0x7F) != 0x7F, "moe_probe_mfma_fp8: code 0x%02x is a NaN", code);
  int st = current_device(nullptr);
  if (st) return st;
  return hip_status(moe::launch_probe_mfma_fp8(n_blocks, iters, code, out, S(stream)),
                    "mfma probe launch");
}

int moe_probe_hbm_read(const void* buf, size_t bytes, int n_blocks, uint32_t* out,
                       void* stream) {
  REQUIRE(buf && out, "moe_probe_hbm_read: null pointer");
  REQUIRE(bytes >= 16 && bytes % 16 == 0, "moe_probe_hbm_read: bytes must be a positive multiple of 16");
  REQUIRE(n_blocks >= 1 && n_blocks <= 65536, "moe_probe_hbm_read: n_blocks must be in [1, 65536]");
  int st = current_device(nullptr);
  if (st) return st;
  return hip_status(moe::launch_probe_read(buf, bytes, n_blocks, out, S(stream)),
                    "read probe launch");
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
  REQUIRE(d->mode == MOE_MODE_FP32 || d->mode == MOE_MODE_FP8 || d->mode == MOE_MODE_W4A16 ||
              d->mode == MOE_MODE_W4A8,
          "moe_layer: unknown mode %d", d->mode);
  REQUIRE(d->route == MOE_ROUTE_SCORE || d->route == MOE_ROUTE_HASH, "moe_layer: unknown route %d",
          d->route);
  REQUIRE(d->route != MOE_ROUTE_HASH || d->k == 1, "moe_layer: hash routing needs k = 1");
  REQUIRE((d->route_flags & ~MOE_ROUTE_RENORM) == 0, "moe_layer: unknown route flags");
  REQUIRE(d->layout == MOE_LAYOUT_CONTIGUOUS || d->layout == MOE_LAYOUT_MASKED,
          "moe_layer: unknown layout %d", d->layout);
  REQUIRE(std::isfinite(d->capacity_factor), "moe_layer: capacity_factor must be finite");
  REQUIRE(d->m_align >= 1 && d->m_align <= 1024, "moe_layer: m_align must be in [1, 1024]");
  REQUIRE(d->d % 128 == 0, "moe_layer: d must be a multiple of 128");
  if (d->mode == MOE_MODE_FP8 || d->mode == MOE_MODE_W4A8) {
    REQUIRE(d->I % 128 == 0, "moe_layer: fp8 needs I %% 128 == 0");
    REQUIRE(d->d <= 128 * moe::kGemmMaxKBlocks && d->I <= 128 * moe::kGemmMaxKBlocks,
            "moe_layer: fp8 needs d, I <= %d", 128 * moe::kGemmMaxKBlocks);
  }
  if (d->mode == MOE_MODE_FP8 || d->mode == MOE_MODE_W4A8) {
    // GEMM1 reads the token codes [T, d], GEMM2 the h codes [R, I] with 32-bit offsets
    const long long R = (long long)d->T * d->k + (long long)d->E * (d->m_align - 1);
    REQUIRE((long long)d->T * d->d <= kMaxOperandBytes && R * d->I <= kMaxOperandBytes,
            "moe_layer: fp8 operands T*d = %lld or rows*I = %lld exceed the 32-bit offset range",
            (long long)d->T * d->d, R * d->I);
  }
  if (d->mode == MOE_MODE_W4A16) REQUIRE(d->I % 128 == 0, "moe_layer: w4a16 needs I %% 128 == 0");
  if (d->mode == MOE_MODE_FP32) REQUIRE(d->I % 16 == 0, "moe_layer: fp32 needs I %% 16 == 0");
  REQUIRE((long long)d->T * d->k + (long long)d->E * (d->m_align - 1) < (1LL << 31),
          "moe_layer: rows bound overflows int32");
  // a positive factor whose capacity floor(ceil(T*k/E) * factor) comes out 0 would drop
  // every slot; the dispatch reads capacity 0 as dropless, so such a factor is refused
  if (d->capacity_factor > 0 && d->T > 0)
    REQUIRE(moe_capacity(d->T, d->k, d->E, d->capacity_factor) >= 1,
            "moe_layer: capacity_factor %g gives capacity floor(ceil(T*k/E) * factor) = 0 "
            "(use a larger factor, or <= 0 for dropless)", d->capacity_factor);
  if (d->layout == MOE_LAYOUT_MASKED) {
    REQUIRE(d->mode == MOE_MODE_FP8, "moe_layer: the masked layout needs MOE_MODE_FP8");
    REQUIRE(d->capacity_factor > 0, "moe_layer: the masked layout needs capacity_factor > 0");
    const int cap = moe_capacity(d->T, d->k, d->E, d->capacity_factor);
    REQUIRE((long long)d->E * cap * std::max(d->d, d->I) <= kMaxOperandBytes,
            "moe_layer: E * capacity rows exceed the 32-bit operand offset range");
  }
  return MOE_OK;
}

// rows of the expert-row buffers: E * capacity (masked) or the contiguous bound
long long layer_rows(const moe_layer_desc* d) {
  if (d->layout == MOE_LAYOUT_MASKED)
    return (long long)d->E * moe_capacity(d->T, d->k, d->E, d->capacity_factor);
  return (long long)moe_rows_bound(d->T, d->k, d->E, d->m_align);
}

LayerWs layer_ws(const moe_layer_desc* d) {
  LayerWs L{};
  const size_t T = d->T, E = d->E, k = d->k, D = d->d, I = d->I;
  const size_t R = (size_t)layer_rows(d);
  const bool masked = d->layout == MOE_LAYOUT_MASKED;
  size_t p = 0;
  auto take = [&](size_t bytes) { size_t at = p; p = align_up(p + bytes); return at; };
  const bool q8 = d->mode == MOE_MODE_FP8 || d->mode == MOE_MODE_W4A8;
  L.part = take(d->route == MOE_ROUTE_SCORE && d->mode != MOE_MODE_FP32
                    ? moe_route_workspace_size(d->T, d->d, d->E, MOE_BF16) : 0);
  L.logits = take(d->route == MOE_ROUTE_SCORE ? T * E * 4 : 0);
  L.idx = take(T * k * 4);
  L.w = take(T * k * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.ros = take(T * k * 4);
  L.sor = take(R * 4);
  if (q8) {
    // masked: the expert-row buffer [E, C, d] of gathered token codes
    L.qx = take((masked ? R : T) * D);
    L.sx = take((masked ? R : T) * (D / 128) * 4);
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

namespace {

// Device pointers of one layer pass inside a workspace region laid out by layer_ws.
struct LayerPtrs {
  float *logits, *part, *gw, *sx, *sh;
  int32_t *idx, *counts, *offsets, *ros, *sor;
  uint8_t *qx, *hq;
  void* o;
};

LayerPtrs layer_ptrs(uint8_t* base, const LayerWs& L, int32_t* counts_out) {
  LayerPtrs P;
  P.logits = reinterpret_cast<float*>(base + L.logits);
  P.part = reinterpret_cast<float*>(base + L.part);
  P.idx = reinterpret_cast<int32_t*>(base + L.idx);
  P.gw = reinterpret_cast<float*>(base + L.w);
  P.counts = counts_out ? counts_out : reinterpret_cast<int32_t*>(base + L.counts);
  P.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  P.ros = reinterpret_cast<int32_t*>(base + L.ros);
  P.sor = reinterpret_cast<int32_t*>(base + L.sor);
  P.qx = base + L.qx;
  P.sx = reinterpret_cast<float*>(base + L.sx);
  P.hq = base + L.h;
  P.sh = reinterpret_cast<float*>(base + L.sh);
  P.o = base + L.o;
  return P;
}

int layer_args(const char* fn, const moe_layer_desc* d, const moe_layer_weights* w, const void* x,
               const int64_t* token_ids, const void* y, const void* ws) {
  int st = layer_check(d);
  if (st) return st;
  REQUIRE(w && ws && ((x && y) || d->T == 0), "%s: null pointer", fn);  // (T = 0: x, y empty)
  REQUIRE(w->w13 && w->w2, "%s: null expert weights", fn);
  if (d->mode != MOE_MODE_FP32) REQUIRE(w->s13 && w->s2, "%s: null weight scales", fn);
  if (d->route == MOE_ROUTE_SCORE)
    REQUIRE(w->w_router && w->bias, "%s: score routing needs w_router and bias", fn);
  else
    REQUIRE(token_ids || d->T == 0, "%s: hash routing needs token_ids", fn);
  return MOE_OK;
}

#define STEP(expr, what) \
  if ((st = hip_status((expr), what))) return st;

// route -> dispatch -> (FP8) token quantisation: everything before the expert GEMMs
int layer_front(const moe_layer_desc* d, const moe_layer_weights* w, const void* x,
                const int64_t* token_ids, const LayerPtrs& P, hipStream_t s) {
  int st = MOE_OK;
  const int T = d->T, D = d->d, E = d->E, k = d->k;
  const int R = (int)layer_rows(d);
  const bool f32 = d->mode == MOE_MODE_FP32;
  const bool masked = d->layout == MOE_LAYOUT_MASKED;
  if (d->route == MOE_ROUTE_SCORE) {
    const int n_part = f32 ? 1 : moe::router_splits(T, D, E, true);
    STEP(moe::launch_router(x, !f32, w->w_router, P.logits, T, D, E, P.part, n_part, s),
         "router launch");
    STEP(moe::launch_topk(P.logits, P.part, n_part, w->bias, T, E, k,
                          d->route_flags & MOE_ROUTE_RENORM, P.idx, P.gw, s),
         "topk launch");
  } else {
    STEP(moe::launch_hash_route(token_ids, T, E, P.idx, P.gw, s), "hash route launch");
  }
  const int cap = moe_capacity(T, k, E, d->capacity_factor);
  if (cap < 0) return cap;
  if (!masked && (d->mode == MOE_MODE_FP8 || d->mode == MOE_MODE_W4A8)) {
    // the per-token quantisation does not depend on the routing: it runs in the dispatch
    // launch, beside the one workgroup that dispatches
    STEP(moe::launch_dispatch_quant(P.idx, T, k, E, d->m_align, cap, P.counts, P.offsets,
                                    P.ros, P.sor, R, x, D, P.qx, P.sx, s),
         "dispatch and quant launch");
    return MOE_OK;
  }
  STEP(moe::launch_dispatch(P.idx, T, k, E, d->m_align, cap, P.counts,
                            masked ? nullptr : P.offsets, P.ros, P.sor, R, s, masked),
       "dispatch launch");
  if (d->mode == MOE_MODE_FP8 && masked) {
    // fixed-capacity layout: token codes gathered into [E, C, d], empty rows zero
    STEP(moe::launch_quant_act(x, true, D, P.sor, k, R, P.qx, P.sx, s), "quant-gather launch");
  }
  return MOE_OK;
}

// grouped GEMM1 (+ SwiGLU) -> grouped GEMM2 -> combine
int layer_back(const moe_layer_desc* d, const moe_layer_weights* w, const void* x,
               const LayerPtrs& P, void* y, int cus, hipStream_t s) {
  int st = MOE_OK;
  const int T = d->T, D = d->d, E = d->E, k = d->k, I = d->I;
  const int R = (int)layer_rows(d);
  const bool f32 = d->mode == MOE_MODE_FP32;
  const bool masked = d->layout == MOE_LAYOUT_MASKED;
  const double rows_per_group = (double)R / E;
  if (d->mode == MOE_MODE_FP8 && masked) {
    // both GEMMs over per-expert row counts clamped to C
    const int cap = R / E;
    STEP(moe::launch_gemm_fp8(P.qx, P.sx, nullptr, 1, static_cast<const uint8_t*>(w->w13),
                              w->s13, P.counts, E, R, I, D, true, P.hq, P.sh, pick_bm(cap), cus,
                              s, moe::kRowsMasked, cap, want_big(cap, D)),
         "masked gemm1 launch");
    STEP(moe::launch_gemm_fp8(P.hq, P.sh, nullptr, 1, static_cast<const uint8_t*>(w->w2), w->s2,
                              P.counts, E, R, D, I, false, P.o, nullptr, pick_bm(cap), cus, s,
                              moe::kRowsMasked, cap, want_big(cap, I)),
         "masked gemm2 launch");
  } else if (d->mode == MOE_MODE_FP8) {
    STEP(moe::launch_gemm_fp8(P.qx, P.sx, P.sor, k, static_cast<const uint8_t*>(w->w13), w->s13,
                              P.offsets, E, R, I, D, true, P.hq, P.sh, pick_bm(rows_per_group),
                              cus, s, moe::kRowsOffsets, 0, want_big(rows_per_group, D)),
         "gemm1 launch");
    STEP(moe::launch_gemm_fp8(P.hq, P.sh, nullptr, 1, static_cast<const uint8_t*>(w->w2), w->s2,
                              P.offsets, E, R, D, I, false, P.o, nullptr,
                              pick_bm(rows_per_group), cus, s, moe::kRowsOffsets, 0,
                              want_big(rows_per_group, I)),
         "gemm2 launch");
  } else if (d->mode == MOE_MODE_W4A8) {
    STEP(moe::launch_gemm_w4a8(P.qx, P.sx, P.sor, k, static_cast<const uint8_t*>(w->w13), w->s13,
                               P.offsets, E, R, I, D, true, P.hq, P.sh, pick_bm(rows_per_group),
                               cus, s),
         "w4a8 gemm1 launch");
    STEP(moe::launch_gemm_w4a8(P.hq, P.sh, nullptr, 1, static_cast<const uint8_t*>(w->w2), w->s2,
                               P.offsets, E, R, D, I, false, P.o, nullptr,
                               pick_bm(rows_per_group), cus, s),
         "w4a8 gemm2 launch");
  } else if (d->mode == MOE_MODE_W4A16) {
    uint16_t* h = reinterpret_cast<uint16_t*>(P.hq);
    STEP(moe::launch_gemm_w4a16(static_cast<const uint16_t*>(x), P.sor, k,
                                static_cast<const uint8_t*>(w->w13), w->s13, P.offsets, E, R, I,
                                D, true, h, cus, s),
         "gemm1 launch");
    STEP(moe::launch_gemm_w4a16(h, nullptr, 1, static_cast<const uint8_t*>(w->w2), w->s2,
                                P.offsets, E, R, D, I, false, static_cast<uint16_t*>(P.o), cus,
                                s),
         "gemm2 launch");
  } else {
    float* h = reinterpret_cast<float*>(P.hq);
    STEP(moe::launch_gemm_f32(static_cast<const float*>(x), P.sor, k,
                              static_cast<const float*>(w->w13), P.offsets, E, R, I, D, true, h,
                              s),
         "gemm1 launch");
    STEP(moe::launch_gemm_f32(h, nullptr, 1, static_cast<const float*>(w->w2), P.offsets, E, R,
                              D, I, false, static_cast<float*>(P.o), s),
         "gemm2 launch");
  }
  STEP(moe::launch_combine(P.o, !f32, P.ros, P.gw, T, k, D, y, !f32, s), "combine launch");
  return MOE_OK;
}

#undef STEP

// the descriptor of the token chunk [t0, t0 + n)
moe_layer_desc chunk_desc(const moe_layer_desc* d, int n) {
  moe_layer_desc c = *d;
  c.T = n;
  return c;
}

}  // namespace

int moe_layer_fwd(const moe_layer_desc* d, const moe_layer_weights* w, const void* x,
                  const int64_t* token_ids, void* y, void* ws, size_t ws_bytes, int32_t* counts_out,
                  void* stream) {
  int st = layer_args("moe_layer_fwd", d, w, x, token_ids, y, ws);
  if (st) return st;
  const LayerWs L = layer_ws(d);
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "moe_layer_fwd: workspace %zu < %zu bytes", ws_bytes, L.total);
  if (d->T == 0) {
    // no tokens: y is empty and every expert's routed count is 0
    if (!counts_out) return MOE_OK;
    if ((st = current_device(nullptr))) return st;
    return hip_status(moe::launch_fill_i32(counts_out, d->E, 0, S(stream)), "fill launch");
  }
  int cus = 0;
  if ((st = current_device(&cus))) return st;
  const LayerPtrs P = layer_ptrs(static_cast<uint8_t*>(ws), L, counts_out);
  if ((st = layer_front(d, w, x, token_ids, P, S(stream)))) return st;
  return layer_back(d, w, x, P, y, cus, S(stream));
}

size_t moe_layer_chunked_workspace_size(const moe_layer_desc* desc, int chunk_tokens) {
  if (layer_check(desc) != MOE_OK) return 0;
  if (chunk_tokens < 1 || desc->capacity_factor > 0 || desc->layout != MOE_LAYOUT_CONTIGUOUS)
    return 0;
  const moe_layer_desc c = chunk_desc(desc, std::min(chunk_tokens, std::max(desc->T, 1)));
  return 2 * align_up(layer_ws(&c).total);
}

int moe_layer_fwd_chunked(const moe_layer_desc* d, const moe_layer_weights* w, const void* x,
                          const int64_t* token_ids, void* y, void* ws, size_t ws_bytes,
                          int chunk_tokens, void* stream, void* stream_aux) {
  int st = layer_args("moe_layer_fwd_chunked", d, w, x, token_ids, y, ws);
  if (st) return st;
  REQUIRE(chunk_tokens >= 1, "moe_layer_fwd_chunked: chunk_tokens must be >= 1");
  REQUIRE(d->capacity_factor <= 0 && d->layout == MOE_LAYOUT_CONTIGUOUS,
          "moe_layer_fwd_chunked: the chunked pipeline is dropless with the contiguous layout");
  REQUIRE(stream != stream_aux, "moe_layer_fwd_chunked: stream_aux must differ from stream");
  const size_t need = moe_layer_chunked_workspace_size(d, chunk_tokens);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_layer_fwd_chunked: workspace %zu < %zu bytes", ws_bytes,
                need);
  if (d->T == 0) return MOE_OK;
  int cus = 0;
  if ((st = current_device(&cus))) return st;
  const hipStream_t sm = S(stream), sa = S(stream_aux);
  const size_t region = need / 2;
  const size_t xb = d->mode == MOE_MODE_FP32 ? 4 : 2;   // bytes per x / y element
  // events: start (main -> aux), front[r] (aux -> main), back[r] (main -> aux), end.
  // Created once per thread and device and reused: a wait already enqueued refers to the
  // record before it, so a later call re-recording the same event does not disturb it.
  int dev = 0;
  if ((st = hip_status(hipGetDevice(&dev), "hipGetDevice"))) return st;
  thread_local hipEvent_t ev_cache[kMaxDevices][6] = {};
  hipEvent_t* ev = ev_cache[dev];
  for (int i = 0; i < 6; ++i)
    if (!ev[i] && (st = hip_status(hipEventCreateWithFlags(&ev[i], hipEventDisableTiming),
                                   "event create")))
      return st;
  hipEvent_t ev_start = ev[0], ev_end = ev[1], ev_front[2] = {ev[2], ev[3]},
             ev_back[2] = {ev[4], ev[5]};
  auto run = [&]() -> int {
    int s2 = MOE_OK;
    // the aux stream starts after the caller's earlier work on the main stream
    if ((s2 = hip_status(hipEventRecord(ev_start, sm), "event record"))) return s2;
    if ((s2 = hip_status(hipStreamWaitEvent(sa, ev_start, 0), "stream wait"))) return s2;
    const int nch = (d->T + chunk_tokens - 1) / chunk_tokens;
    for (int i = 0; i < nch; ++i) {
      const int t0 = i * chunk_tokens, n = std::min(chunk_tokens, d->T - t0), r = i & 1;
      const moe_layer_desc c = chunk_desc(d, n);
      const LayerWs L = layer_ws(&c);
      const LayerPtrs P = layer_ptrs(static_cast<uint8_t*>(ws) + r * region, L, nullptr);
      const void* xc = static_cast<const uint8_t*>(x) + (size_t)t0 * d->d * xb;
      void* yc = static_cast<uint8_t*>(y) + (size_t)t0 * d->d * xb;
      const int64_t* ids = token_ids ? token_ids + t0 : nullptr;
      // region r was last read by chunk i-2's GEMMs and combine
      if (i >= 2 && (s2 = hip_status(hipStreamWaitEvent(sa, ev_back[r], 0), "stream wait")))
        return s2;
      if ((s2 = layer_front(&c, w, xc, ids, P, sa))) return s2;
      if ((s2 = hip_status(hipEventRecord(ev_front[r], sa), "event record"))) return s2;
      if ((s2 = hip_status(hipStreamWaitEvent(sm, ev_front[r], 0), "stream wait"))) return s2;
      if ((s2 = layer_back(&c, w, xc, P, yc, cus, sm))) return s2;
      if ((s2 = hip_status(hipEventRecord(ev_back[r], sm), "event record"))) return s2;
    }
    // the caller's stream ends after everything either stream was given
    if ((s2 = hip_status(hipEventRecord(ev_end, sa), "event record"))) return s2;
    return hip_status(hipStreamWaitEvent(sm, ev_end, 0), "stream wait");
  };
  return run();
}

}  // extern "C"
