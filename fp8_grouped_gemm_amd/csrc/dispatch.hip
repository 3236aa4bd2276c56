// Dispatch: expert histogram, padded exclusive scan and stable slot -> row scatter.
//
// Tokens routed to one expert are concatenated into one contiguous block of rows
// (expert grouping, MegaMoE walkthrough, discosf.com sec. 2.1), each block padded
// to a multiple of m_align so the grouped GEMM's row tiles stay inside one expert.
// An optional capacity keeps the first C slots of each expert and drops the rest
// silently (DeepSeek MoE architecture, mooersco.com sec. 2.5).  In the fixed-capacity
// ("masked") layout every expert owns exactly C rows, expert e rows [e C, e C + C)
// whatever its count (the second grouped layout of DeepGEMM, qidao123.com day 3).
//
// Ranks come from integer counts and lane masks only, so the result does not depend on
// scheduling.  Up to 512 experts one workgroup does it all (dispatch_fused_kernel);
// above that, one workgroup per expert scans the whole slot list.
#include "common.hpp"
#include "launch.hpp"
#include "quant_act.hpp"

namespace moe {

namespace {
__device__ __forceinline__ int block_sum_256(int v, int* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) red[wid] = v;
  __syncthreads();
  int total = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return total;
}
}  // namespace

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx,
                                                             int n_slots,
                                                             int32_t* __restrict__ counts) {
  __shared__ int red[4];
  const int e = blockIdx.x;
  int c = 0;
  for (int s = threadIdx.x; s < n_slots; s += 256) c += (idx[s] == e);
  c = block_sum_256(c, red);
  if (threadIdx.x == 0) counts[e] = c;
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, int n_slots, int E, int m_align, int cap, bool fixed,
    const int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_of_slot, int32_t* __restrict__ slot_of_row, int rows_bound) {
  __shared__ int red[4];
  __shared__ int wave_cnt[4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

  // offsets[e] and offsets[E] from the padded kept counts of every expert
  int before = 0, all = 0;
  for (int j = tid; j < E; j += 256) {
    int kept = cap > 0 ? min(counts[j], cap) : counts[j];
    int padded = fixed ? cap : (kept + m_align - 1) / m_align * m_align;
    all += padded;
    if (j < e) before += padded;
  }
  before = block_sum_256(before, red);
  all = block_sum_256(all, red);
  if (tid == 0 && offsets) {
    offsets[e] = before;
    if (e == E - 1) offsets[E] = all;
  }
  const int cnt = counts[e];
  const int kept = cap > 0 ? min(cnt, cap) : cnt;
  const int padded = fixed ? cap : (kept + m_align - 1) / m_align * m_align;

  // stable scatter: rank of each matching slot = matches before it in slot order
  int running = 0;
  for (int base = 0; base < n_slots; base += 256) {
    const int s = base + tid;
    const bool match = s < n_slots && idx[s] == e;
    const unsigned long long mask = __ballot(match);
    if (lane == 0) wave_cnt[wid] = __popcll(mask);
    __syncthreads();
    int prefix = running;
    for (int w = 0; w < wid; ++w) prefix += wave_cnt[w];
    prefix += __popcll(mask & ((1ull << lane) - 1ull));
    const int total = wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    __syncthreads();
    if (match) {
      if (prefix < kept) {
        const int row = before + prefix;
        row_of_slot[s] = row;
        slot_of_row[row] = s;
      } else {
        row_of_slot[s] = -1;
      }
    }
    running += total;
    if (running >= cnt) break;  // uniform across the block
  }
  for (int r = kept + tid; r < padded; r += 256) slot_of_row[before + r] = -1;
  // rows past the last expert: split across the workgroups
  for (int r = all + e * 256 + tid; r < rows_bound; r += E * 256) slot_of_row[r] = -1;
}

// One workgroup of 16 waves.  Wave w owns the contiguous slot segment [w S, (w+1) S).
// Pass 1 counts each segment's slots per expert; a scan over experts (padded kept
// counts) gives the offsets, and a scan over the segments of each expert turns the
// counts into each segment's first row.  Pass 2 walks every segment in order, 64 slots
// at a time: a 64-bit mask per expert marks the lanes that chose it, so a slot's rank
// among them is the popcount of the mask below its lane, and the lowest such lane
// advances the expert's row.  Slot order inside every expert is thus preserved.
//
// QX: workgroups 1.. quantise the token rows (bf16 x [T, K] -> 1x128 e4m3 codes and
// scales, 64 blocks of 128 per workgroup) while workgroup 0 dispatches: the quantisation
// does not depend on the routing, and the dispatch alone occupies one CU.
struct QuantRows {
  const void* x;
  int K, rows;
  uint8_t* q;
  float* scales;
};

template <int EMAX, bool QX = false>
__global__ __launch_bounds__(1024) void dispatch_fused_kernel(
    const int32_t* __restrict__ idx, int n_slots, int E, int m_align, int cap, bool fixed,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_of_slot, int32_t* __restrict__ slot_of_row, int rows_bound,
    QuantRows qr = {}) {
  if constexpr (QX) {
    if (blockIdx.x > 0) {
      const int KB = qr.K / 128;
      const long g = ((long)(blockIdx.x - 1) * 1024 + threadIdx.x) >> 4;
      if (g >= (long)qr.rows * KB) return;     // whole 16-lane groups exit together
      const int row = (int)(g / KB), kb = (int)(g % KB);
      quant_act_block<true>(qr.x, qr.K, row, row, kb, threadIdx.x & 15, qr.q, qr.scales);
      return;
    }
  }
  constexpr int NW = 16;
  __shared__ int cnt[NW][EMAX];                    // counts, then running row of the segment
  __shared__ unsigned long long msk[NW][EMAX];
  __shared__ int off_s[EMAX + 1], kept_s[EMAX];
  __shared__ int wsum[NW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < NW * EMAX; i += 1024) {
    (&cnt[0][0])[i] = 0;
    (&msk[0][0])[i] = 0ull;
  }
  for (int r = tid; r < rows_bound; r += 1024) slot_of_row[r] = -1;
  __syncthreads();
  const int seg = (n_slots + NW - 1) / NW;
  const int s0 = min(w * seg, n_slots), s1 = min(s0 + seg, n_slots);
  for (int s = s0 + lane; s < s1; s += 64) {
    const int e = idx[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[w][e], 1);   // other values: dropped
  }
  __syncthreads();

  // experts: totals, kept and padded counts, exclusive scan of the padded counts
  int total = 0, padded = 0;
  if (tid < E) {
#pragma unroll
    for (int v = 0; v < NW; ++v) total += cnt[v][tid];
    const int kept = cap > 0 ? min(total, cap) : total;
    padded = fixed ? cap : (kept + m_align - 1) / m_align * m_align;
    kept_s[tid] = kept;
    counts[tid] = total;
  }
  int incl = padded;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0;
  for (int v = 0; v < w; ++v) before += wsum[v];
  const int excl = before + incl - padded;
  if (tid < E) {
    off_s[tid] = excl;
    if (offsets) offsets[tid] = excl;
    int run = excl;                                // first row of each segment's slots
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const int c = cnt[v][tid];
      cnt[v][tid] = run;
      run += c;
    }
  }
  if (tid == E - 1) {
    off_s[E] = excl + padded;
    if (offsets) offsets[E] = excl + padded;
  }
  __syncthreads();

  const unsigned long long below = (1ull << lane) - 1ull;
  for (int sb = s0; sb < s1; sb += 64) {
    const int s = sb + lane;
    const int e = s < s1 ? idx[s] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    if (s < s1 && !valid) row_of_slot[s] = -1;
    if (valid) atomicOr(&msk[w][e], 1ull << lane);
    const unsigned long long m = valid ? msk[w][e] : 0ull;
    const int row = valid ? cnt[w][e] + __popcll(m & below) : 0;
    // the wave's LDS accesses run in order: every lane has read the mask and the row
    // before the lowest lane of each expert advances and clears them
    if (valid && (m & below) == 0ull) {
      cnt[w][e] += __popcll(m);
      msk[w][e] = 0ull;
    }
    if (valid) {
      if (row - off_s[e] < kept_s[e]) {
        row_of_slot[s] = row;
        slot_of_row[row] = s;
      } else {
        row_of_slot[s] = -1;
      }
    }
  }
}

hipError_t launch_dispatch(const int32_t* idx, int T, int k, int E, int m_align, int cap,
                           int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                           int32_t* slot_of_row, int rows_bound, hipStream_t s, bool fixed) {
  const int n = T * k;
  if (E <= 256) {
    hipLaunchKernelGGL(dispatch_fused_kernel<256>, dim3(1), dim3(1024), 0, s, idx, n, E, m_align,
                       cap, fixed, counts, offsets, row_of_slot, slot_of_row, rows_bound);
    return hipGetLastError();
  }
  if (E <= 512) {
    hipLaunchKernelGGL(dispatch_fused_kernel<512>, dim3(1), dim3(1024), 0, s, idx, n, E, m_align,
                       cap, fixed, counts, offsets, row_of_slot, slot_of_row, rows_bound);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(E), dim3(256), 0, s, idx, n, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(E), dim3(256), 0, s, idx, n, E, m_align, cap,
                     fixed, counts, offsets, row_of_slot, slot_of_row, rows_bound);
  return hipGetLastError();
}

hipError_t launch_dispatch_quant(const int32_t* idx, int T, int k, int E, int m_align, int cap,
                                 int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                                 int32_t* slot_of_row, int rows_bound, const void* x, int K,
                                 uint8_t* q, float* scales, hipStream_t s) {
  if (E > 512 || T == 0) {
    hipError_t err = launch_dispatch(idx, T, k, E, m_align, cap, counts, offsets, row_of_slot,
                                     slot_of_row, rows_bound, s);
    if (err != hipSuccess) return err;
    return launch_quant_act(x, true, K, nullptr, 1, T, q, scales, s);
  }
  const QuantRows qr{x, K, T, q, scales};
  const long qblocks = ((long)T * (K / 128) * 16 + 1023) / 1024;
  const dim3 grid((unsigned)(1 + qblocks)), block(1024);
  const int n = T * k;
  if (E <= 256)
    hipLaunchKernelGGL((dispatch_fused_kernel<256, true>), grid, block, 0, s, idx, n, E, m_align,
                       cap, false, counts, offsets, row_of_slot, slot_of_row, rows_bound, qr);
  else
    hipLaunchKernelGGL((dispatch_fused_kernel<512, true>), grid, block, 0, s, idx, n, E, m_align,
                       cap, false, counts, offsets, row_of_slot, slot_of_row, rows_bound, qr);
  return hipGetLastError();
}

// n int32 values set to v (a kernel rather than a memset node, so that a captured graph
// replays it like the other kernels)
__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int n, int v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace moe
