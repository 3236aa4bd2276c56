// Weighted combine: y[t] = sum_j w[t,j] * o[row_of_slot[t*k+j]] (the top-k weighted sum
// y = sum_i G(x)_i E_i(x), MegaMoE walkthrough, discosf.com sec. 2.1).
//
// A gather, not a scatter: each token reads its k expert rows and sums them in fp32
// in slot order j = 0..k-1, so the result is deterministic (no atomics).  One
// workgroup per token; each thread handles 8 consecutive columns (16-byte bf16 loads).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

template <bool OBF16, bool YBF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ o,
                                                      const int32_t* __restrict__ row_of_slot,
                                                      const float* __restrict__ w, int k, int d,
                                                      void* __restrict__ y) {
  const int t = blockIdx.x;
  const int chunks = d / 8;
  for (int c = threadIdx.x; c < chunks; c += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int row = row_of_slot[(size_t)t * k + j];
      if (row < 0) continue;
      const float wj = w[(size_t)t * k + j];
      float v[8];
      if (OBF16) {
        v4i raw = *reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(o) +
                                                 (size_t)row * d + c * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = bf16_to_f32((uint16_t)(raw[i] & 0xFFFF));
          v[2 * i + 1] = bf16_to_f32((uint16_t)((uint32_t)raw[i] >> 16));
        }
      } else {
        const float* p = static_cast<const float*>(o) + (size_t)row * d + c * 8;
        v4f a = *reinterpret_cast<const v4f*>(p);
        v4f b = *reinterpret_cast<const v4f*>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
    }
    if (YBF16) {
      v4i out;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[i] = (int)((uint32_t)f32_to_bf16(acc[2 * i]) |
                       ((uint32_t)f32_to_bf16(acc[2 * i + 1]) << 16));
      *reinterpret_cast<v4i*>(static_cast<uint16_t*>(y) + (size_t)t * d + c * 8) = out;
    } else {
      float* p = static_cast<float*>(y) + (size_t)t * d + c * 8;
      *reinterpret_cast<v4f*>(p) = v4f{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<v4f*>(p + 4) = v4f{acc[4], acc[5], acc[6], acc[7]};
    }
  }
}

hipError_t launch_combine(const void* o, bool o_bf16, const int32_t* row_of_slot,
                          const float* w, int T, int k, int d, void* y, bool y_bf16,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid(T), block(256);
  if (o_bf16 && y_bf16)
    hipLaunchKernelGGL((combine_kernel<true, true>), grid, block, 0, s, o, row_of_slot, w, k, d, y);
  else if (o_bf16)
    hipLaunchKernelGGL((combine_kernel<true, false>), grid, block, 0, s, o, row_of_slot, w, k, d, y);
  else if (y_bf16)
    hipLaunchKernelGGL((combine_kernel<false, true>), grid, block, 0, s, o, row_of_slot, w, k, d, y);
  else
    hipLaunchKernelGGL((combine_kernel<false, false>), grid, block, 0, s, o, row_of_slot, w, k, d, y);
  return hipGetLastError();
}

}  // namespace moe
