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
hipError_t launch_hash_route(const int64_t* ids, int T, int E, int32_t* idx, float* w,
                             hipStream_t s);
hipError_t launch_dispatch(const int32_t* idx, int T, int k, int E, int m_align, int cap,
                           int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                           int32_t* slot_of_row, int rows_bound, hipStream_t s);
hipError_t launch_quant_act(const void* x, bool bf16, int K, const int32_t* src_row, int src_div,
                            int rows_out, uint8_t* q, float* scales, hipStream_t s);
hipError_t launch_quant_weight_fp8(const float* w, int G, int N, int K, uint8_t* q,
                                   float* scales, hipStream_t s);
hipError_t launch_quant_weight_int4(const float* w, int G, int N, int K, uint8_t* q, float* s7,
                                    hipStream_t s);
// The FP8 GEMM keeps a tile's activation scales for every K block in LDS: K <= 128 * this.
constexpr int kGemmMaxKBlocks = 128;
// B [G][R][K] e4m3 -> the fragment-major layout the FP8 GEMM reads (same byte count)
hipError_t launch_pack_weight_fp8(const uint8_t* B, int G, int R, int K, uint8_t* Bf,
                                  hipStream_t s);
// bm: rows per tile of small groups (16, 32, 64; larger values mean 64); Bf is
// fragment-major (launch_pack_weight_fp8)
hipError_t launch_gemm_fp8(const uint8_t* A, const float* sA, const int32_t* a_rows,
                           int a_row_div, const uint8_t* B, const float* sB,
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
hipError_t launch_combine(const void* o, bool o_bf16, const int32_t* row_of_slot,
                          const float* w, int T, int k, int d, void* y, bool y_bf16,
                          hipStream_t s);

}  // namespace moe
