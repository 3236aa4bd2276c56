// Measurement probes: the rate the FP8 matrix core and the HBM read path actually reach
// on the device the library runs on, as references beside the datasheet peaks.  They
// are not part of the layer's computation.
//
//   * probe_mfma_fp8_kernel: every wave issues `iters` rounds of four independent
//     16x16x128 e4m3 MFMAs (the instruction the FP8 GEMMs issue, called the same way;
//     four accumulators, so no MFMA waits for the previous one's result) on register
//     operands whose bytes all hold one e4m3 code.  Run at 512 threads per workgroup and
//     one workgroup per CU, two waves per SIMD, as the GEMMs run.  The output (each
//     lane's sum of its 16 accumulator values) is checkable: 4 * 4 * 128 * iters * v^2
//     for the code's value v.
//   * probe_read_kernel: a grid-strided read of a buffer with 16-byte non-temporal loads,
//     four in flight per thread, XOR-folded so that every loaded word is used; one 32-bit
//     XOR per workgroup is written.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

__global__ __launch_bounds__(512, 1) void probe_mfma_fp8_kernel(int iters, uint32_t code,
                                                                float* out) {
  const int w = (int)(code * 0x01010101u);
  const v8i a = {w, w, w, w, w, w, w, w};
  v4f c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, c0, 0, 0, 0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, c1, 0, 0, 0, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, c2, 0, 0, 0, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, c3, 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(512) void probe_read_kernel(const v4i* __restrict__ buf, size_t n16,
                                                         uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const v4i v0 = __builtin_nontemporal_load(buf + i);
    const v4i v1 = __builtin_nontemporal_load(buf + i + stride);
    const v4i v2 = __builtin_nontemporal_load(buf + i + 2 * stride);
    const v4i v3 = __builtin_nontemporal_load(buf + i + 3 * stride);
    x ^= (uint32_t)(v0[0] ^ v0[1] ^ v0[2] ^ v0[3] ^ v1[0] ^ v1[1] ^ v1[2] ^ v1[3]);
    x ^= (uint32_t)(v2[0] ^ v2[1] ^ v2[2] ^ v2[3] ^ v3[0] ^ v3[1] ^ v3[2] ^ v3[3]);
  }
  for (; i < n16; i += stride) {
    const v4i v = __builtin_nontemporal_load(buf + i);
    x ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  __shared__ uint32_t ws[8];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) ws[wid] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) r ^= ws[k];
    out[blockIdx.x] = r;
  }
}

hipError_t launch_probe_mfma_fp8(int n_blocks, int iters, uint32_t code, float* out,
                                 hipStream_t s) {
  hipLaunchKernelGGL(probe_mfma_fp8_kernel, dim3((unsigned)n_blocks), dim3(512), 0, s, iters,
                     code, out);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* buf, size_t bytes, int n_blocks, uint32_t* out,
                             hipStream_t s) {
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)n_blocks), dim3(512), 0, s,
                     static_cast<const v4i*>(buf), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace moe
