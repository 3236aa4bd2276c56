// Routing kernels: router logits (bf16 MFMA or fp32 VALU), biased fp32 softmax with
// wave-level top-k, and hash routing.
//
// The gate is one linear layer followed by softmax(W_g x + b) (MegaMoE walkthrough,
// discosf.com sec. 2.2) computed in fp32 (DeepSeek-V4 lecture, tqpw.cn sec. 2.3).
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace moe {

// ---------------------------------------------------------------- router GEMM
// logits[T, E] = x[T, d] . W[E, d]^T with bf16 inputs and fp32 accumulation on the
// 16x16x32 bf16 MFMA.  Workgroup tile 128 tokens x 256 experts, 8 waves as 2 x 4 wave
// tiles of 64 x 64.  64-deep K chunks of both operands reach LDS by DMA into three
// stages (separate LDS objects), two chunks ahead, one barrier per chunk.  With split-K
// every workgroup sums its range of chunks into partial plane blockIdx.z; the top-k
// kernel adds the planes in plane order.
namespace {
constexpr int RT_BM = 128, RT_BN = 256, RT_BK = 64;   // BK in elements: 128-byte rows
constexpr int RT_SA = RT_BM * 128, RT_SB = RT_BN * 128;   // stage bytes per operand
constexpr int RT_ADMA = RT_BM / 8 / 8, RT_BDMA = RT_BN / 8 / 8;   // DMAs per wave per chunk
constexpr int RT_MIN_CHUNKS = 4;                      // per workgroup under split-K

// XOR key of the 16-byte pieces of a 128-byte LDS row.  A fragment read hands the 16
// lanes the LDS serves together ({0-7, 16-23}, ...) rows r..r+7 at pieces q and q+1
// (q even); keys 0, 2, 4, 6 over the four rows of one parity keep them in 16 banks groups.
__device__ __forceinline__ int rt_key(int r) { return ((r >> 1) & 3) << 1; }
}  // namespace

__global__ __launch_bounds__(512, 1) void router_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ logits,
    int T, int d, int E, int chunks_per_split) {
  __shared__ __attribute__((aligned(1024))) uint8_t sa0[RT_SA];
  __shared__ __attribute__((aligned(1024))) uint8_t sa1[RT_SA];
  __shared__ __attribute__((aligned(1024))) uint8_t sa2[RT_SA];
  __shared__ __attribute__((aligned(1024))) uint8_t sb0[RT_SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sb1[RT_SB];
  __shared__ __attribute__((aligned(1024))) uint8_t sb2[RT_SB];
  auto stage_a = [&](auto S) -> uint8_t* {
    constexpr int i = decltype(S)::value % 3;
    if constexpr (i == 0) return sa0;
    else if constexpr (i == 1) return sa1;
    else return sa2;
  };
  auto stage_b = [&](auto S) -> uint8_t* {
    constexpr int i = decltype(S)::value % 3;
    if constexpr (i == 0) return sb0;
    else if constexpr (i == 1) return sb1;
    else return sb2;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 2, wn = wid & 3;
  const int t0 = blockIdx.x * RT_BM, e0 = blockIdx.y * RT_BN;
  const int c0 = blockIdx.z * chunks_per_split;
  const int nc = min(chunks_per_split, d / RT_BK - c0);   // >= 1 by the launcher
  logits += (size_t)blockIdx.z * T * E;

  // DMA instruction q of a wave fills 8 rows (1 KB) of group wid + 8 q: lane L lands at
  // row L/8, slot L%8 and fetches piece (L%8) ^ rt_key(row).  Rows past T or E repeat
  // the last one; their results are not stored.
  const uint8_t* xa = reinterpret_cast<const uint8_t*>(x + (size_t)t0 * d + (size_t)c0 * RT_BK);
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(w + (size_t)e0 * d + (size_t)c0 * RT_BK);
  uint32_t a_off[RT_ADMA], b_off[RT_BDMA];
#pragma unroll
  for (int q = 0; q < RT_ADMA; ++q) {
    const int row = (wid + 8 * q) * 8 + (lane >> 3), slot = lane & 7;
    a_off[q] = (uint32_t)(min(t0 + row, T - 1) - t0) * (uint32_t)(d * 2) +
               ((slot ^ rt_key(row)) << 4);
  }
#pragma unroll
  for (int q = 0; q < RT_BDMA; ++q) {
    const int row = (wid + 8 * q) * 8 + (lane >> 3), slot = lane & 7;
    b_off[q] = (uint32_t)(min(e0 + row, E - 1) - e0) * (uint32_t)(d * 2) +
               ((slot ^ rt_key(row)) << 4);
  }
  // chunk c (clamped to the last one, so every call issues the same DMA count)
  auto dma = [&](auto S, int c) {
    const size_t cb = (size_t)min(c, nc - 1) * (RT_BK * 2);
    uint8_t* la = stage_a(S);
    uint8_t* lb = stage_b(S);
#pragma unroll
    for (int q = 0; q < RT_ADMA; ++q) dma16b(xa + cb, a_off[q], la + (wid + 8 * q) * 1024);
#pragma unroll
    for (int q = 0; q < RT_BDMA; ++q) dma16b(wb + cb, b_off[q], lb + (wid + 8 * q) * 1024);
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // chunk c in stage c % 3: wait for this wave's DMA of it (one chunk's DMAs came after),
  // barrier (everyone's DMA of c landed, everyone done with c - 1), refill the stage of
  // c - 1 with c + 2, then 2 K steps of 32
  auto body = [&](auto U, int c) {
    wait_vmcnt<RT_ADMA + RT_BDMA>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    dma(std::integral_constant<int, decltype(U)::value + 2>{}, c + 2);
    const uint8_t* la = stage_a(U);
    const uint8_t* lb = stage_b(U);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int piece = ks * 4 + (lane >> 4);     // 8 bf16
      v8bf af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = wm * 64 + i * 16 + (lane & 15);
        const int rb = wn * 64 + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const v8bf*>(la + ra * 128 + ((piece ^ rt_key(ra)) << 4));
        bf[i] = *reinterpret_cast<const v8bf*>(lb + rb * 128 + ((piece ^ rt_key(rb)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };
  dma(std::integral_constant<int, 0>{}, 0);
  dma(std::integral_constant<int, 1>{}, 1);
  int c = 0;
  for (; c + 3 <= nc; c += 3)
    static_for<3>([&](auto U) { body(U, c + decltype(U)::value); });
  static_for<2>([&](auto U) {
    if (c + decltype(U)::value < nc) body(U, c + decltype(U)::value);
  });
  wait_vmcnt<0>();   // the clamped repeat DMAs land before the workgroup's LDS is freed

  // C layout of a 16x16 MFMA tile: lane holds column lane%16, rows 4*(lane/16)+r.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = e0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = t0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
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
  float key[KPL], l[KPL];
  bool live[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    live[i] = lane + 64 * i < E;
    l[i] = 0.f;
  }
  if (n_part > 1) {
    // sum the planes in plane order, eight planes' loads in flight at a time
    const float* pp = part + (size_t)t * E + lane;
    const size_t ps = (size_t)T * E;
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (live[i]) l[i] = pp[64 * i];
    for (int s0 = 1; s0 < n_part; s0 += 8) {
      float v[8][KPL];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < KPL; ++i)
          v[u][i] = (s0 + u < n_part && live[i]) ? pp[(size_t)(s0 + u) * ps + 64 * i] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < n_part) {
#pragma unroll
          for (int i = 0; i < KPL; ++i) l[i] += v[u][i];
        }
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (live[i]) row[lane + 64 * i] = l[i];
  } else {
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (live[i]) l[i] = row[lane + 64 * i];
  }
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = live[i] ? l[i] + (bias ? bias[e] : 0.0f) : -INFINITY;
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

// ------------------------------------------------------------- static scratch
// Device memory of the allocation-free router entry point: the split-K partial planes.
// One copy per GPU, alive until the process ends; kernels reach it through the address
// hipGetSymbolAddress returns on that GPU (the array's name is not a device address in
// host code).  Every call on a GPU shares it, so overlapping calls on one GPU race.
namespace {
static __device__ __align__(256) uint8_t scratch[kRouteScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];
}  // namespace

hipError_t route_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// ------------------------------------------------------------------ launchers
int router_splits(int T, int d, int E, bool bf16) {
  if (!bf16) return 1;
  // about one workgroup per CU, each with at least RT_MIN_CHUNKS chunks
  const long tiles = (long)((T + RT_BM - 1) / RT_BM) * ((E + RT_BN - 1) / RT_BN);
  const int chunks = d / RT_BK;
  const int most = std::max(1, chunks / RT_MIN_CHUNKS);
  const int want = (int)std::min<long>(std::max<long>(1, 256 / tiles), most);
  const int cps = (chunks + want - 1) / want;
  return (chunks + cps - 1) / cps;
}

hipError_t launch_router(const void* x, bool bf16, const void* w, float* logits, int T, int d,
                         int E, float* part, int n_part, hipStream_t s) {
  if (bf16) {
    // n_part planes of ceil(chunks / n_part) chunks; every plane gets at least one
    const int chunks = d / RT_BK;
    const int cps = (chunks + n_part - 1) / n_part;
    if (n_part < 1 || (long)(n_part - 1) * cps >= chunks) return hipErrorInvalidValue;
    dim3 grid((T + RT_BM - 1) / RT_BM, (E + RT_BN - 1) / RT_BN, n_part);
    hipLaunchKernelGGL(router_bf16_kernel, grid, dim3(512), 0, s,
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
