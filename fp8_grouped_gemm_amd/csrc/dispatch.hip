// Dispatch: expert histogram, padded exclusive scan and stable slot -> row scatter.
//
// Tokens routed to one expert are concatenated into one contiguous block of rows
// (expert grouping, MegaMoE walkthrough, discosf.com sec. 2.1), each block padded
// to a multiple of m_align so the grouped GEMM's row tiles stay inside one expert.
// An optional capacity keeps the first C slots of each expert and drops the rest
// silently (DeepSeek MoE architecture, mooersco.com sec. 2.5).
//
// One workgroup per expert scans the whole slot list in order, so ranks come from
// integer prefix counts only: the result does not depend on scheduling.
#include "common.hpp"
#include "launch.hpp"

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
    const int32_t* __restrict__ idx, int n_slots, int E, int m_align, int cap,
    const int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_of_slot, int32_t* __restrict__ slot_of_row, int rows_bound) {
  __shared__ int red[4];
  __shared__ int wave_cnt[4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

  // offsets[e] and offsets[E] from the padded kept counts of every expert
  int before = 0, all = 0;
  for (int j = tid; j < E; j += 256) {
    int kept = cap > 0 ? min(counts[j], cap) : counts[j];
    int padded = (kept + m_align - 1) / m_align * m_align;
    all += padded;
    if (j < e) before += padded;
  }
  before = block_sum_256(before, red);
  all = block_sum_256(all, red);
  if (tid == 0) {
    offsets[e] = before;
    if (e == E - 1) offsets[E] = all;
  }
  const int cnt = counts[e];
  const int kept = cap > 0 ? min(cnt, cap) : cnt;
  const int padded = (kept + m_align - 1) / m_align * m_align;

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

hipError_t launch_dispatch(const int32_t* idx, int T, int k, int E, int m_align, int cap,
                           int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                           int32_t* slot_of_row, int rows_bound, hipStream_t s) {
  const int n = T * k;
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(E), dim3(256), 0, s, idx, n, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(E), dim3(256), 0, s, idx, n, E, m_align, cap,
                     counts, offsets, row_of_slot, slot_of_row, rows_bound);
  return hipGetLastError();
}

}  // namespace moe
