// Weighted combine: y[t] = sum_j w[t,j] * o[row_of_slot[t*k+j]] (the top-k weighted sum
// y = sum_i G(x)_i E_i(x), MegaMoE walkthrough, discosf.com sec. 2.1).
//
// A gather, not a scatter: each token reads its k expert rows and sums them in fp32
// in slot order j = 0..k-1, so the result is deterministic (no atomics).  One
// workgroup per token; each thread handles 8 consecutive columns (16-byte loads).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// the k rows of a chunk summed in slot order (the same order and roundings whatever the
// batching below); o row loads of one batch are all issued before the first add
template <bool OBF16, int KU>
__device__ __forceinline__ void add_rows(const void* __restrict__ o, const int* rows,
                                         const float* wv, int n, int d, int c, float* acc) {
  constexpr int VW = OBF16 ? 1 : 2;               // 16-byte loads per slot and chunk
  v4i raw[KU][VW];
#pragma unroll
  for (int u = 0; u < KU; ++u) {                  // slots past n or dropped read row 0
    const size_t r = (size_t)max(u < n ? rows[u] : 0, 0);
    if (OBF16) {
      const v4i* p = reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(o) + r * d + c * 8);
      // each o row is read once: with four or more rows per token the loads are
      // non-temporal (prefill, k = 8: 108 -> 96 us; with one row per token they measured
      // slower, 21 -> 24 us)
      raw[u][0] = KU >= 4 ? __builtin_nontemporal_load(p) : *p;
    } else {
      const float* p = static_cast<const float*>(o) + r * d + c * 8;
      raw[u][0] = *reinterpret_cast<const v4i*>(p);
      raw[u][VW - 1] = *reinterpret_cast<const v4i*>(p + 4);
    }
  }
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    if (u >= n || rows[u] < 0) continue;          // the same for the whole workgroup
    float v[8];
    if (OBF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32((uint16_t)(raw[u][0][i] & 0xFFFF));
        v[2 * i + 1] = bf16_to_f32((uint16_t)((uint32_t)raw[u][0][i] >> 16));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = __int_as_float(raw[u][0][i]);
        v[4 + i] = __int_as_float(raw[u][VW - 1][i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wv[u], v[i], acc[i]);
  }
}

template <bool OBF16, bool YBF16, int KU>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ o,
                                                      const int32_t* __restrict__ row_of_slot,
                                                      const float* __restrict__ w, int k, int d,
                                                      void* __restrict__ y) {
  // KU: slots per batch of loads (the launcher picks the smallest of 1, 2, 4, 8 that
  // holds k, or 8 with batches for larger k)
  const int t = blockIdx.x;
  const int chunks = d / 8;
  // k <= KU: the token's rows and weights once, in scalar registers
  int rows0[KU];
  float w0[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int jc = min(u, k - 1);
    rows0[u] = row_of_slot[(size_t)t * k + jc];
    w0[u] = w[(size_t)t * k + jc];
  }
  for (int c = threadIdx.x; c < chunks; c += 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (k <= KU) {
      add_rows<OBF16, KU>(o, rows0, w0, k, d, c, acc);
    } else {
      for (int j0 = 0; j0 < k; j0 += KU) {
        int rows[KU];
        float wv[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
          const int jc = min(j0 + u, k - 1);
          rows[u] = row_of_slot[(size_t)t * k + jc];
          wv[u] = w[(size_t)t * k + jc];
        }
        add_rows<OBF16, KU>(o, rows, wv, min(KU, k - j0), d, c, acc);
      }
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

template <int KU>
void launch_combine_ku(const void* o, bool o_bf16, const int32_t* row_of_slot, const float* w,
                       int T, int k, int d, void* y, bool y_bf16, hipStream_t s) {
  dim3 grid(T), block(256);
  if (o_bf16 && y_bf16)
    hipLaunchKernelGGL((combine_kernel<true, true, KU>), grid, block, 0, s, o, row_of_slot, w,
                       k, d, y);
  else if (o_bf16)
    hipLaunchKernelGGL((combine_kernel<true, false, KU>), grid, block, 0, s, o, row_of_slot, w,
                       k, d, y);
  else if (y_bf16)
    hipLaunchKernelGGL((combine_kernel<false, true, KU>), grid, block, 0, s, o, row_of_slot, w,
                       k, d, y);
  else
    hipLaunchKernelGGL((combine_kernel<false, false, KU>), grid, block, 0, s, o, row_of_slot,
                       w, k, d, y);
}

hipError_t launch_combine(const void* o, bool o_bf16, const int32_t* row_of_slot,
                          const float* w, int T, int k, int d, void* y, bool y_bf16,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (k == 1)
    launch_combine_ku<1>(o, o_bf16, row_of_slot, w, T, k, d, y, y_bf16, s);
  else if (k == 2)
    launch_combine_ku<2>(o, o_bf16, row_of_slot, w, T, k, d, y, y_bf16, s);
  else if (k <= 4)
    launch_combine_ku<4>(o, o_bf16, row_of_slot, w, T, k, d, y, y_bf16, s);
  else
    launch_combine_ku<8>(o, o_bf16, row_of_slot, w, T, k, d, y, y_bf16, s);
  return hipGetLastError();
}

}  // namespace moe
