// Host-side launchers of the gfx950 kernels (internal to the library).  Each one
// enqueues its kernels on `s` and returns hipGetLastError(); arguments were checked
// by the C ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// split-K planes the router uses for this shape (1 = no split, partials unused)
int router_splits(int T, int d, int E, bool bf16);
hipError_t launch_router(const void* x, bool bf16, const void* w, float* logits, int T, int d,
                         int E, float* part, int n_part, hipStream_t s);
// n_part > 1: logits are the plane-order sums of part[n_part][T][E], written by this call
hipError_t launch_topk(float* logits, const float* part, int n_part, const float* bias, int T,
                       int E, int k, bool renorm, int32_t* idx, float* w, hipStream_t s);
// Bytes of the router's static device scratch (split-K partial planes of the
// allocation-free entry point) and its address on the current device.
constexpr size_t kRouteScratchBytes = size_t(32) << 20;
hipError_t route_scratch(void** ptr);
hipError_t launch_hash_route(const int64_t* ids, int T, int E, int32_t* idx, float* w,
                             hipStream_t s);
// fixed: the masked layout, every expert owning exactly cap rows (offsets may be null)
hipError_t launch_dispatch(const int32_t* idx, int T, int k, int E, int m_align, int cap,
                           int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                           int32_t* slot_of_row, int rows_bound, hipStream_t s,
                           bool fixed = false);
// launch_dispatch (contiguous layout) and launch_quant_act of bf16 x [T, K] (no gather) in
// one launch: one workgroup dispatches while the others quantise (E <= 512; above that
// the two launches)
hipError_t launch_dispatch_quant(const int32_t* idx, int T, int k, int E, int m_align, int cap,
                                 int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                                 int32_t* slot_of_row, int rows_bound, const void* x, int K,
                                 uint8_t* q, float* scales, hipStream_t s);
// p[0..n) = v
hipError_t launch_fill_i32(int32_t* p, int n, int v, hipStream_t s);
hipError_t launch_quant_act(const void* x, bool bf16, int K, const int32_t* src_row, int src_div,
                            int rows_out, uint8_t* q, float* scales, hipStream_t s);
hipError_t launch_quant_weight_fp8(const float* w, int G, int N, int K, uint8_t* q,
                                   float* scales, hipStream_t s);
hipError_t launch_quant_weight_int4(const float* w, int G, int N, int K, uint8_t* q, float* s7,
                                    hipStream_t s);
// The FP8 GEMM keeps a tile's activation scales for every K block in LDS: K <= 128 * this.
constexpr int kGemmMaxKBlocks = 128;
// ... and its 192-row tiles (three stages of 24 KB beside the table) for K <= 128 * this
constexpr int kGemmMaxKBlocks192 = 64;
// B [G][R][K] e4m3 -> the fragment-major layout the FP8 GEMM reads (same byte count)
hipError_t launch_pack_weight_fp8(const uint8_t* B, int G, int R, int K, uint8_t* Bf,
                                  hipStream_t s);
// bm: rows per tile of small groups (16, 32, 64; larger values mean 64); Bf is
// fragment-major (launch_pack_weight_fp8)
// big: the whole 256-row tiles of large groups, in whole rounds of the grid, go to a
// 256 x 256-tile kernel launched first (N a multiple of 256, or SwiGLU); the rest of every
// group to the 128-row / small-tile kernel after it
hipError_t launch_gemm_fp8(const uint8_t* A, const float* sA, const int32_t* a_rows,
                           int a_row_div, const uint8_t* B, const float* sB,
                           const int32_t* offsets, int G, int R_cap, int N, int K, bool swiglu,
                           void* C, float* sC, int bm, int num_cus, hipStream_t s,
                           int rows_mode = 0, int cap = 0, bool big = false);
// rows of the FP8 GEMM's large-group tiles (128 or 192) for a launch (gemm_fp8.hip)
int large_tile_rows(int rows_mode, int M, int N, int K, bool swiglu, int num_cus, bool big);
// the 256 x 256-tile kernel alone, and its row tiles per round (the cut both launches use)
int big_rows_per_round(int N, bool swiglu, int num_cus);
hipError_t launch_gemm_fp8_big(const uint8_t* A, const float* sA, const int32_t* a_rows,
                               int a_row_div, const uint8_t* Bf, const float* sB,
                               const int32_t* offsets, int G, int N, int K, bool swiglu, void* C,
                               float* sC, int num_cus, hipStream_t s, int rows_mode, int cap);
// int4 codes [G][R][K/2] and scales [G][R][K/128] -> the fragment-major order the W4A8
// GEMM loads: codes [G][R/16][K/128][64][16 B], scales [G][R/16][K/128][16]
hipError_t launch_pack_weight_int4(const uint8_t* q, const float* s7, int G, int R, int K,
                                   uint8_t* qf, float* s7f, hipStream_t s);
// the FP8 GEMM with packed 4-bit weights (W4A8); arguments as launch_gemm_fp8
hipError_t launch_gemm_w4a8(const uint8_t* A, const float* sA, const int32_t* a_rows,
                            int a_row_div, const uint8_t* Bf, const float* s7f,
                            const int32_t* offsets, int G, int R_cap, int N, int K, bool swiglu,
                            void* C, float* sC, int bm, int num_cus, hipStream_t s,
                            int rows_mode = 0, int cap = 0);
hipError_t launch_gemm_w4a16(const uint16_t* A, const int32_t* a_rows, int a_row_div,
                             const uint8_t* B, const float* s7, const int32_t* offsets, int G,
                             int R_cap, int N, int K, bool swiglu, uint16_t* C, int num_cus,
                             hipStream_t s);
hipError_t launch_gemm_f32(const float* A, const int32_t* a_rows, int a_row_div, const float* B,
                           const int32_t* offsets, int G, int R_cap, int N, int K, bool swiglu,
                           float* C, hipStream_t s);
// measurement probes (probe.hip): n_blocks workgroups of 512 threads each
hipError_t launch_probe_mfma_fp8(int n_blocks, int iters, uint32_t code, float* out,
                                 hipStream_t s);
hipError_t launch_probe_read(const void* buf, size_t bytes, int n_blocks, uint32_t* out,
                             hipStream_t s);
hipError_t launch_combine(const void* o, bool o_bf16, const int32_t* row_of_slot,
                          const float* w, int T, int k, int d, void* y, bool y_bf16,
                          hipStream_t s);

}  // namespace moe
