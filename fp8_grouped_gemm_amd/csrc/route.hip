// Routing kernels: router logits (bf16 MFMA or fp32 VALU), biased fp32 softmax with
// wave-level top-k, and hash routing.
//
// The gate is one linear layer followed by softmax(W_g x + b) (MegaMoE walkthrough,
// discosf.com sec. 2.2) computed in fp32 (DeepSeek-V4 lecture, tqpw.cn sec. 2.3).
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

// ---------------------------------------------------------------- router GEMM
// logits[T, E] = x[T, d] . W[E, d]^T with bf16 inputs and fp32 accumulation on the
// 16x16x32 bf16 MFMA.  Workgroup tile 64 tokens x 64 experts, 4 waves as 2x2 of
// 32x32; K staged through LDS in 128-wide chunks, two chunks in flight in registers.
namespace {
constexpr int RT_BM = 64, RT_BN = 64, RT_BK = 128;      // BK in elements
constexpr int RT_ROWB = RT_BK * 2;                        // 256 bytes per row per chunk
constexpr int RT_CPR = RT_ROWB / 16;                      // 16-byte pieces per row: 16
constexpr int RT_LOADS = RT_BM * RT_CPR / 256;            // per thread per operand: 4
}  // namespace

__global__ __launch_bounds__(256) void router_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ logits,
    int T, int d, int E, int chunks_per_split) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][RT_BM * RT_ROWB];  // [A|B][row*256]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int m0 = blockIdx.x * RT_BM, n0 = blockIdx.y * RT_BN;
  const int wm = wid >> 1, wn = wid & 1;
  // split-K: this workgroup sums K chunks [c0, c0 + nchunk) into partial plane blockIdx.z
  const int c0 = blockIdx.z * chunks_per_split;
  const int nchunk = min(chunks_per_split, d / RT_BK - c0);
  logits += (size_t)blockIdx.z * T * E;

  const uint8_t* a_ptr[RT_LOADS];
  const uint8_t* b_ptr[RT_LOADS];
  int lds_off[RT_LOADS];
#pragma unroll
  for (int i = 0; i < RT_LOADS; ++i) {
    int c = tid + i * 256;
    int row = c / RT_CPR, piece = c % RT_CPR;
    int ar = min(m0 + row, T - 1), br = min(n0 + row, E - 1);
    a_ptr[i] = reinterpret_cast<const uint8_t*>(x + (size_t)ar * d + (size_t)c0 * RT_BK) + piece * 16;
    b_ptr[i] = reinterpret_cast<const uint8_t*>(w + (size_t)br * d + (size_t)c0 * RT_BK) + piece * 16;
    lds_off[i] = row * RT_ROWB + ((piece ^ (row & 15)) * 16);
  }
  v4i ra[2][RT_LOADS], rb[2][RT_LOADS];
  auto issue = [&](int slot, int ch) {
#pragma unroll
    for (int i = 0; i < RT_LOADS; ++i) {
      ra[slot][i] = *reinterpret_cast<const v4i*>(a_ptr[i] + (size_t)ch * RT_ROWB);
      rb[slot][i] = *reinterpret_cast<const v4i*>(b_ptr[i] + (size_t)ch * RT_ROWB);
    }
  };
  v4f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  if (nchunk > 1) issue(1, 1);
  for (int ch = 0; ch < nchunk; ++ch) {
    const int slot = ch & 1;
#pragma unroll
    for (int i = 0; i < RT_LOADS; ++i) {
      *reinterpret_cast<v4i*>(&lds[0][lds_off[i]]) = ra[slot][i];
      *reinterpret_cast<v4i*>(&lds[1][lds_off[i]]) = rb[slot][i];
    }
    __syncthreads();
    if (ch + 2 < nchunk) issue(slot, ch + 2);
#pragma unroll
    for (int ks = 0; ks < RT_BK / 32; ++ks) {
      v8bf af[2], bf[2];
      const int piece = ks * 4 + (lane >> 4);              // 8 bf16 = one 16-byte piece
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int ar = wm * 32 + i * 16 + (lane & 15);
        int br = wn * 32 + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const v8bf*>(&lds[0][ar * RT_ROWB + ((piece ^ (ar & 15)) * 16)]);
        bf[i] = *reinterpret_cast<const v8bf*>(&lds[1][br * RT_ROWB + ((piece ^ (br & 15)) * 16)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // C layout of a 16x16 MFMA tile: lane holds column lane%16, rows 4*(lane/16)+r.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int col = n0 + wn * 32 + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int row = m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
        if (row < T && col < E) logits[(size_t)row * E + col] = acc[i][j][r];
      }
    }
}

// fp32 router: one thread per (token, expert) dot product (small layers).
__global__ __launch_bounds__(256) void router_f32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ w,
                                                         float* __restrict__ logits, int T,
                                                         int d, int E) {
  int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T * E) return;
  int t = i / E, e = i % E;
  const float* xr = x + (size_t)t * d;
  const float* wr = w + (size_t)e * d;
  float acc = 0.f;
  for (int c = 0; c < d; ++c) acc = fmaf(xr[c], wr[c], acc);
  logits[i] = acc;
}

// ---------------------------------------------------------------------- top-k
// One wave per token.  Keys key_e = fl32(logit_e + b_e) live KPL per lane (expert
// e = lane + 64*i).  k rounds of a wave arg-max pick the largest key, the lower
// expert index winning ties; the softmax over all E keys is taken in fp32.
// With n_part > 1 the logits arrive as split-K partial planes part[n_part][T][E]; they
// are summed here in plane order (deterministic) and the sums written to logits.
template <int KPL>
__global__ __launch_bounds__(256) void topk_kernel(float* __restrict__ logits,
                                                   const float* __restrict__ part, int n_part,
                                                   const float* __restrict__ bias, int T,
                                                   int E, int k, int renorm,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float* row = logits + (size_t)t * E;
  float key[KPL];
  bool live[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    int e = lane + 64 * i;
    live[i] = e < E;
    float l = 0.f;
    if (live[i]) {
      if (n_part > 1) {
        const float* pp = part + (size_t)t * E + e;
        l = pp[0];
        for (int s = 1; s < n_part; ++s) l += pp[(size_t)s * T * E];
        row[e] = l;
      } else {
        l = row[e];
      }
    }
    key[i] = live[i] ? l + (bias ? bias[e] : 0.0f) : -INFINITY;
  }
  // softmax denominator over every expert
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < KPL; ++i) m = fmaxf(m, key[i]);
  m = group_max<64>(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < KPL; ++i) s += live[i] ? expf(key[i] - m) : 0.0f;
  s = group_sum<64>(s);
  const float inv = 1.0f / s;

  float chosen_p = 0.f, psum = 0.f;
  for (int j = 0; j < k; ++j) {
    // lane-local best among live keys
    float bk = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      int e = lane + 64 * i;
      if (live[i] && (key[i] > bk || (key[i] == bk && e < be))) { bk = key[i]; be = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      float ok = __shfl_xor(bk, o, 64);
      int oe = __shfl_xor(be, o, 64);
      if (ok > bk || (ok == bk && oe < be)) { bk = ok; be = oe; }
    }
    float p = expf(bk - m) * inv;
    if (lane == j) chosen_p = p;
    psum += p;
    if ((be & 63) == lane) {
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if (lane + 64 * i == be) live[i] = false;
    }
    if (lane == 0) idx[(size_t)t * k + j] = be;
  }
  if (lane < k) wout[(size_t)t * k + lane] = renorm ? chosen_p / psum : chosen_p;
}

// ---------------------------------------------------------------------- hash
// expert = ((id * 2654435761) mod 2^32) mod E, weight 1 (tqpw.cn sec. 2.2).
__global__ void hash_route_kernel(const int64_t* __restrict__ ids, int T, int E,
                                  int32_t* __restrict__ idx, float* __restrict__ w) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  uint32_t h = (uint32_t)((uint64_t)ids[t] * 2654435761ull);
  idx[t] = (int32_t)(h % (uint32_t)E);
  w[t] = 1.0f;
}

// ------------------------------------------------------------------ launchers
int router_splits(int T, int d, int E, bool bf16) {
  if (!bf16) return 1;
  const long tiles = (long)((T + RT_BM - 1) / RT_BM) * ((E + RT_BN - 1) / RT_BN);
  const int chunks = d / RT_BK;
  int want = (int)std::min<long>(std::max<long>(1, (1024 + tiles - 1) / tiles), chunks);
  const int cps = (chunks + want - 1) / want;
  return (chunks + cps - 1) / cps;
}

hipError_t launch_router(const void* x, bool bf16, const void* w, float* logits, int T, int d,
                         int E, float* part, int n_part, hipStream_t s) {
  if (bf16) {
    const int chunks = d / RT_BK;
    const int cps = (chunks + n_part - 1) / n_part;
    dim3 grid((T + RT_BM - 1) / RT_BM, (E + RT_BN - 1) / RT_BN, n_part);
    hipLaunchKernelGGL(router_bf16_kernel, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                       n_part > 1 ? part : logits, T, d, E, cps);
  } else {
    int n = T * E;
    hipLaunchKernelGGL(router_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, s,
                       static_cast<const float*>(x), static_cast<const float*>(w), logits, T, d,
                       E);
  }
  return hipGetLastError();
}

hipError_t launch_topk(float* logits, const float* part, int n_part, const float* bias, int T,
                       int E, int k, bool renorm, int32_t* idx, float* w, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  int r = renorm ? 1 : 0;
#define MOE_TOPK(KPL) \
  hipLaunchKernelGGL(topk_kernel<KPL>, grid, block, 0, s, logits, part, n_part, bias, T, E, k, \
                     r, idx, w)
  if (E <= 64) MOE_TOPK(1);
  else if (E <= 128) MOE_TOPK(2);
  else if (E <= 256) MOE_TOPK(4);
  else if (E <= 512) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

hipError_t launch_hash_route(const int64_t* ids, int T, int E, int32_t* idx, float* w,
                             hipStream_t s) {
  hipLaunchKernelGGL(hash_route_kernel, dim3((T + 255) / 256), dim3(256), 0, s, ids, T, E, idx,
                     w);
  return hipGetLastError();
}

}  // namespace moe
