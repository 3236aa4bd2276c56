// Persistent tile scheduling over per-group row ranges, shared by the grouped GEMMs.
//
// Groups own row ranges given one of three ways (GroupRows): contiguous, from prefix
// offsets [offsets[g], offsets[g+1]); fixed-capacity ("masked"), rows [g C, g C +
// counts[g]) of a [G, C] row block per group; dense, a single group of M rows.  Each
// group is cut into ceil(M_g / BM) row tiles and every row tile into tiles_n column
// tiles.  Tiles are numbered group by group (a flattened tile list over all groups, as
// the global tile scheduler in the MegaMoE walkthrough, discosf.com sec. 3.2,
// describes).  A split map keeps two such lists: the large groups' row tiles (start)
// and the small groups' single row tiles (sstart), for kernels that interleave them.
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kMaxGroups = 1024;


enum GroupRows { kRowsOffsets = 0, kRowsMasked = 1, kRowsDense = 2 };

// Tile bookkeeping shared by the workgroup: per-group row-tile prefix sums.
struct TileMap {
  int start[kMaxGroups + 1];  // first row tile of each group (exclusive prefix)
  int sstart[kMaxGroups + 1]; // split maps: first small-group tile (start: large groups)
  int off[kMaxGroups + 1];    // offsets: copy; masked: counts clamped to [0, C]; dense: 0, M
  int mode, cap;              // GroupRows and C (masked) or M (dense)
};

// first row and row count of group g, before any rows are handed to a 256-row-tile launch
__device__ __forceinline__ int group_row0_all(const TileMap& tm, int g) {
  return tm.mode == kRowsMasked ? g * tm.cap : tm.off[g];
}
__device__ __forceinline__ int group_rows_all(const TileMap& tm, int g) {
  return tm.mode == kRowsMasked ? tm.off[g] : tm.off[g + 1] - tm.off[g];
}
// the rows this launch handles: skip (an LDS array, or null) holds each group's leading
// rows that a 256-row-tile launch handles
__device__ __forceinline__ int group_row0(const TileMap& tm, int g, const int* skip = nullptr) {
  return group_row0_all(tm, g) + (skip ? skip[g] : 0);
}
__device__ __forceinline__ int group_rows(const TileMap& tm, int g, const int* skip = nullptr) {
  return group_rows_all(tm, g) - (skip ? skip[g] : 0);
}

// Exclusive prefix over groups of count(g) into pre[0..G] (pre[G] = the total), by the
// NT threads of the workgroup; every thread must call it.
template <int NT, typename F>
__device__ void group_prefix(int* pre, int G, F count) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  __shared__ int ws[NW];
  const int per = (G + NT - 1) / NT;
  const int g0 = min(tid * per, G), g1 = min(g0 + per, G);
  int local = 0;
  for (int g = g0; g < g1; ++g) local += count(g);
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) ws[wid] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wid; ++w) base += ws[w];
  int run = base + incl - local;
  for (int g = g0; g < g1; ++g) {
    pre[g] = run;
    run += count(g);
  }
  if (tid == NT - 1) pre[G] = base + incl;
  __syncthreads();
}

// Rows of 256-row tiles: a group of M rows holds M / 256 whole ones.  A launch of those
// tiles takes whole rounds of its grid: the first cut row tiles in group order, cut =
// total rounded down to a multiple of rpr (row tiles per round; rpr = 0: all of them).
constexpr int kBigRows = 256;
__device__ __forceinline__ int big_cut(int total, int rpr) {
  return rpr > 0 ? total / rpr * rpr : total;
}

// Rows per tile of a group with M rows: BMS for small groups (M <= BMS), BMB otherwise.
template <int BMS, int BMB>
__device__ __forceinline__ int tile_rows(int M) { return M <= BMS ? BMS : BMB; }

// big_rpr >= 0 (with an LDS array skip_buf of G + 1 ints): the leading whole 256-row
// tiles that a 256-row-tile launch with that many row tiles per round takes (big_cut)
// are skipped here.
template <int BMS, int BMB = BMS, int NT = 256, bool SPLIT = false>
__device__ void build_tile_map(TileMap& tm, const int32_t* __restrict__ offsets, int G,
                               int mode = kRowsOffsets, int cap = 0, int big_rpr = -1,
                               int* skip_buf = nullptr) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  __shared__ int wsum[NW], wsum2[NW];
  const bool split = big_rpr >= 0 && skip_buf;
  const int* skip = split ? skip_buf : nullptr;
  if (tid == 0) {
    tm.mode = mode;
    tm.cap = cap;
  }
  for (int i = tid; i <= G; i += NT) {
    if (mode == kRowsOffsets) tm.off[i] = offsets[i];
    else if (mode == kRowsMasked) tm.off[i] = i < G ? min(max(offsets[i], 0), cap) : 0;
    else tm.off[i] = i == 0 ? 0 : cap;
  }
  __syncthreads();
  if (split) {
    // the 256-row-tile launch's prefix, kept in start until the tile counts replace it
    group_prefix<NT>(tm.start, G, [&](int g) { return group_rows_all(tm, g) / kBigRows; });
    const int cut = big_cut(tm.start[G], big_rpr);
    for (int g = tid; g < G; g += NT) {
      const int nb = group_rows_all(tm, g) / kBigRows;
      skip_buf[g] = kBigRows * min(max(cut - tm.start[g], 0), nb);
    }
    __syncthreads();
  }
  // each thread owns a contiguous chunk of groups
  const int per = (G + NT - 1) / NT;
  const int g0 = min(tid * per, G), g1 = min(g0 + per, G);
  // row tiles of group g: all of them (combined map) or, for a split map, the large
  // groups' (first) and the small groups' (second)
  auto count = [&](int g, int& big, int& small) {
    const int M = group_rows(tm, g, skip);
    if (SPLIT) {
      big = M > BMS ? (M + BMB - 1) / BMB : 0;
      small = (M > 0 && M <= BMS) ? 1 : 0;
    } else {
      const int bm = tile_rows<BMS, BMB>(M);
      big = (M + bm - 1) / bm;
      small = 0;
    }
  };
  int local = 0, local2 = 0;
  for (int g = g0; g < g1; ++g) {
    int b, s;
    count(g, b, s);
    local += b;
    local2 += s;
  }
  int incl = local, incl2 = local2;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int v = __shfl_up(incl, o, 64), v2 = __shfl_up(incl2, o, 64);
    if (lane >= o) {
      incl += v;
      incl2 += v2;
    }
  }
  if (lane == 63) {
    wsum[wid] = incl;
    wsum2[wid] = incl2;
  }
  __syncthreads();
  int base = 0, base2 = 0;
  for (int w = 0; w < wid; ++w) {
    base += wsum[w];
    base2 += wsum2[w];
  }
  int run = base + incl - local, run2 = base2 + incl2 - local2;
  for (int g = g0; g < g1; ++g) {
    tm.start[g] = run;
    if (SPLIT) tm.sstart[g] = run2;
    int b, s;
    count(g, b, s);
    run += b;
    run2 += s;
  }
  if (tid == NT - 1) {
    tm.start[G] = base + incl;
    if (SPLIT) tm.sstart[G] = base2 + incl2;
  }
  __syncthreads();
}

// largest g in [0, G) with start[g] * tiles_n <= t
__device__ __forceinline__ int find_group(const int* start, int G, int t, int tiles_n) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (start[mid] * tiles_n <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}
__device__ __forceinline__ int find_group(const TileMap& tm, int G, int t, int tiles_n) {
  return find_group(tm.start, G, t, tiles_n);
}

}  // namespace moe
