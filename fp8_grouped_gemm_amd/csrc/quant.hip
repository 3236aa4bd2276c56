// Quantisers: per-row 1x128 e4m3 activations (with an optional row gather), 128x128
// e4m3 weight blocks, and 1x128 per-channel int4 weight blocks.
//
// e4m3: x_q = clamp(round(x / scale), -448, 448) (MegaMoE walkthrough, discosf.com
// sec. 3.3) with one scale per block (fine-grained scaling, DeepGEMM release notes,
// qidao123.com day 3): scale = amax / 448, so the block's largest element maps to 448.
// int4: W_q = round(W / scale_block * 7), scale_block = block max-abs (DeepSeek-V4
// lecture, tqpw.cn sec. 3.1).
#include "common.hpp"
#include "launch.hpp"
#include "quant_act.hpp"

namespace moe {

// 16 lanes per 128-wide block, 8 elements per lane.
template <bool BF16>
__global__ __launch_bounds__(256) void quant_act_kernel(const void* __restrict__ x, int K,
                                                        const int32_t* __restrict__ src_row,
                                                        int src_div, int rows_out,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ scales) {
  const int KB = K / 128;
  const long g = ((long)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int li = threadIdx.x & 15;
  if (g >= (long)rows_out * KB) return;   // whole 16-lane groups exit together
  const int row = (int)(g / KB), kb = (int)(g % KB);
  int src = row;
  if (src_row) {
    int sr = src_row[row];
    src = sr < 0 ? -1 : sr / src_div;
  }
  quant_act_block<BF16>(x, K, src, row, kb, li, q, scales);
}

// One workgroup per 128x128 block: thread t owns row t/2, 64 consecutive elements.
__global__ __launch_bounds__(256) void quant_weight_fp8_kernel(const float* __restrict__ w,
                                                               int N, int K,
                                                               uint8_t* __restrict__ q,
                                                               float* __restrict__ scales) {
  __shared__ float red[4];
  const int KB = K / 128, NB = N / 128;
  const int kb = blockIdx.x, nb = blockIdx.y, g = blockIdx.z;
  const int tid = threadIdx.x, r = tid >> 1, half = tid & 1;
  const size_t base = ((size_t)g * N + (size_t)nb * 128 + r) * K + (size_t)kb * 128 + half * 64;
  float v[64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v4f t = *reinterpret_cast<const v4f*>(w + base + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[4 * i + j] = t[j];
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<64>(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = block_scale(amax);
  uint32_t out[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    out[i] = e4m3x4(clamp448(v[4 * i] / s), clamp448(v[4 * i + 1] / s),
                    clamp448(v[4 * i + 2] / s), clamp448(v[4 * i + 3] / s));
  v4i* qp = reinterpret_cast<v4i*>(q + base);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    qp[i] = v4i{(int)out[4 * i], (int)out[4 * i + 1], (int)out[4 * i + 2], (int)out[4 * i + 3]};
  if (tid == 0) scales[((size_t)g * NB + nb) * KB + kb] = s;
}

// 16 lanes per (row, 128-wide block), 8 elements per lane -> 4 packed bytes.
__global__ __launch_bounds__(256) void quant_weight_int4_kernel(const float* __restrict__ w,
                                                                long rows, int K,
                                                                uint8_t* __restrict__ q,
                                                                float* __restrict__ s7) {
  const int KB = K / 128;
  const long g = ((long)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int li = threadIdx.x & 15;
  if (g >= rows * KB) return;
  const long row = g / KB;
  const int kb = (int)(g % KB);
  const float* p = w + row * K + kb * 128 + li * 8;
  v4f a = *reinterpret_cast<const v4f*>(p);
  v4f b = *reinterpret_cast<const v4f*>(p + 4);
  float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<16>(amax);
  if (amax == 0.f) amax = 1.f;
  // one 32-bit word per 8 codes: byte b holds code b (low nibble) and code 4 + b (high),
  // each nibble sign (bit 3) and magnitude
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float t = v[i] / amax;
    t = t * 7.0f;
    const int qi = (int)rintf(t);
    const uint32_t nib = qi < 0 ? (8u | (uint32_t)(-qi)) : (uint32_t)qi;
    packed |= nib << (8 * (i & 3) + 4 * (i >> 2));
  }
  *reinterpret_cast<uint32_t*>(q + row * (K / 2) + kb * 64 + li * 4) = packed;
  if (li == 0) s7[row * KB + kb] = amax / 7.0f;
}

hipError_t launch_quant_act(const void* x, bool bf16, int K, const int32_t* src_row, int src_div,
                            int rows_out, uint8_t* q, float* scales, hipStream_t s) {
  const long groups = (long)rows_out * (K / 128);
  const long blocks = (groups * 16 + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(quant_act_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, x, K,
                       src_row, src_div, rows_out, q, scales);
  else
    hipLaunchKernelGGL(quant_act_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, x, K,
                       src_row, src_div, rows_out, q, scales);
  return hipGetLastError();
}

hipError_t launch_quant_weight_fp8(const float* w, int G, int N, int K, uint8_t* q, float* scales,
                                   hipStream_t s) {
  hipLaunchKernelGGL(quant_weight_fp8_kernel, dim3(K / 128, N / 128, G), dim3(256), 0, s, w, N, K,
                     q, scales);
  return hipGetLastError();
}

hipError_t launch_quant_weight_int4(const float* w, int G, int N, int K, uint8_t* q, float* s7,
                                    hipStream_t s) {
  const long rows = (long)G * N;
  const long blocks = (rows * (K / 128) * 16 + 255) / 256;
  hipLaunchKernelGGL(quant_weight_int4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, rows, K,
                     q, s7);
  return hipGetLastError();
}

}  // namespace moe
