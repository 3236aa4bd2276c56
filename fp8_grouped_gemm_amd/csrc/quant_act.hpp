// 1x128 e4m3 quantisation of one activation block, shared by the quantiser kernel and
// the dispatch kernel's quantising blocks: x_q = clamp(round(x / scale), -448, 448) with
// scale = amax / 448 (MegaMoE walkthrough, discosf.com sec. 3.3; one scale per 1x128
// block, DeepGEMM's fine-grained scaling, qidao123.com day 3).
#pragma once
#include "common.hpp"

namespace moe {

// Block kb of output row `row`, read from input row `src` (src < 0: an empty row, zeros
// with scale 1) by the 16 lanes li = 0..15 of an aligned lane group, 8 consecutive
// elements each.  Every lane of the group must call it (the block maximum is a 16-lane
// reduction).
template <bool BF16>
__device__ __forceinline__ void quant_act_block(const void* __restrict__ x, int K, int src,
                                                int row, int kb, int li,
                                                uint8_t* __restrict__ q,
                                                float* __restrict__ scales) {
  const int KB = K / 128;
  float v[8];
  if (src < 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  } else if (BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(x) + (size_t)src * K + kb * 128 + li * 8;
    v4i raw = *reinterpret_cast<const v4i*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32((uint16_t)(raw[i] & 0xFFFF));
      v[2 * i + 1] = bf16_to_f32((uint16_t)((uint32_t)raw[i] >> 16));
    }
  } else {
    const float* p = static_cast<const float*>(x) + (size_t)src * K + kb * 128 + li * 8;
    v4f a = *reinterpret_cast<const v4f*>(p);
    v4f b = *reinterpret_cast<const v4f*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<16>(amax);
  const float s = block_scale(amax);
  uint32_t lo = e4m3x4(clamp448(v[0] / s), clamp448(v[1] / s), clamp448(v[2] / s),
                       clamp448(v[3] / s));
  uint32_t hi = e4m3x4(clamp448(v[4] / s), clamp448(v[5] / s), clamp448(v[6] / s),
                       clamp448(v[7] / s));
  uint32_t* qp = reinterpret_cast<uint32_t*>(q + (size_t)row * K + kb * 128 + li * 8);
  qp[0] = lo;
  qp[1] = hi;
  if (li == 0) scales[(size_t)row * KB + kb] = s;
}

}  // namespace moe
