// Persistent tile scheduling over per-group row offsets, shared by the grouped GEMMs.
//
// Groups own row ranges [offsets[g], offsets[g+1]); each is cut into ceil(M_g / BM)
// row tiles and every row tile into tiles_n column tiles.  Tiles are numbered group
// by group, column tile by column tile, row tile fastest, so that consecutive tiles
// share one B column tile (a flattened tile list over all groups, as the global tile
// scheduler in the MegaMoE walkthrough, discosf.com sec. 3.2, describes).
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kMaxGroups = 1024;


// Tile bookkeeping shared by the workgroup: per-group row-tile prefix sums.
struct TileMap {
  int start[kMaxGroups + 1];  // first row tile of each group (exclusive prefix)
  int off[kMaxGroups + 1];    // copy of offsets
};

// Rows per tile of a group with M rows: BMS for small groups (M <= BMS), BMB otherwise.
template <int BMS, int BMB>
__device__ __forceinline__ int tile_rows(int M) { return M <= BMS ? BMS : BMB; }

template <int BMS, int BMB = BMS, int NT = 256>
__device__ void build_tile_map(TileMap& tm, const int32_t* __restrict__ offsets, int G) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  __shared__ int wsum[NW];
  for (int i = tid; i <= G; i += NT) tm.off[i] = offsets[i];
  __syncthreads();
  // each thread owns a contiguous chunk of groups
  const int per = (G + NT - 1) / NT;
  const int g0 = min(tid * per, G), g1 = min(g0 + per, G);
  int local = 0;
  for (int g = g0; g < g1; ++g) {
    const int M = tm.off[g + 1] - tm.off[g];
    const int bm = tile_rows<BMS, BMB>(M);
    local += (M + bm - 1) / bm;
  }
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wid; ++w) base += wsum[w];
  int run = base + incl - local;
  for (int g = g0; g < g1; ++g) {
    tm.start[g] = run;
    const int M = tm.off[g + 1] - tm.off[g];
    const int bm = tile_rows<BMS, BMB>(M);
    run += (M + bm - 1) / bm;
  }
  if (tid == NT - 1) tm.start[G] = base + incl;
  __syncthreads();
}

// largest g in [0, G) with start[g] * tiles_n <= t
__device__ __forceinline__ int find_group(const TileMap& tm, int G, int t, int tiles_n) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (tm.start[mid] * tiles_n <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace moe
