// Grouped fp32 GEMM (no quantisation) with an optional fused SwiGLU: the plain
// per-group product of the grouped GEMM definition (MegaMoE walkthrough, discosf.com
// sec. 3.2), used for fp32 layers.  Workgroup = 16 rows x 64 columns, one thread per
// (row, 4 columns); every row looks up its own group, so any row padding works.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const int32_t* __restrict__ a_rows,
                                                       int a_row_div, const float* __restrict__ B,
                                                       const int32_t* __restrict__ offsets,
                                                       int G, int N, int K,
                                                       float* __restrict__ C) {
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c0 = blockIdx.y * 64 + (threadIdx.x & 15);
  if (row >= offsets[G]) return;
  int lo = 0, hi = G - 1;  // group of this row: largest g with offsets[g] <= row
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  int src = row;
  if (a_rows) {
    int sr = a_rows[row];
    src = sr < 0 ? 0 : sr / a_row_div;
  }
  const float* a = A + (size_t)src * K;
  const size_t nb = SWIGLU ? 2 * (size_t)N : (size_t)N;
  const float* b = B + (size_t)g * nb * K;
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, accu[4] = {0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < K; ++kk) {
    const float av = a[kk];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = c0 + 16 * q;
      if (col < N) {
        acc[q] = fmaf(av, b[(size_t)col * K + kk], acc[q]);
        if (SWIGLU) accu[q] = fmaf(av, b[(size_t)(N + col) * K + kk], accu[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int col = c0 + 16 * q;
    if (col < N) C[(size_t)row * N + col] = SWIGLU ? silu(acc[q]) * accu[q] : acc[q];
  }
}

hipError_t launch_gemm_f32(const float* A, const int32_t* a_rows, int a_row_div, const float* B,
                           const int32_t* offsets, int G, int R_cap, int N, int K, bool swiglu,
                           float* C, hipStream_t s) {
  dim3 grid((R_cap + 15) / 16, (N + 63) / 64), block(256);
  if (grid.x == 0) return hipSuccess;
  if (swiglu)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, grid, block, 0, s, A, a_rows, a_row_div, B, offsets,
                       G, N, K, C);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, block, 0, s, A, a_rows, a_row_div, B, offsets,
                       G, N, K, C);
  return hipGetLastError();
}

}  // namespace moe
