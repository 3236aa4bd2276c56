// Grouped FP8 GEMM kernel for gfx950 (template shared by the e4m3-weight and int4-weight
// instances): C[rows of g] = A[rows of g] . B[g]^T with e4m3 operands,
// 1x128 activation scales and 128x128 weight scales.
//
// What it computes (MegaMoE walkthrough, discosf.com sec. 3.2): groups differ in M
// and share N and K; a global tile scheduler flattens every group's row tiles into
// one list so small and large groups keep the machine busy.  Each 128-deep K block
// is reduced by the FP8 matrix core into a fresh fp32 partial and then promoted into
// the fp32 accumulator with its two scales (the two-level accumulation of DeepGEMM's
// release notes, qidao123.com day 3).  The output is rounded to bf16 (RNE, walkthrough
// sec. 3.3) or, with the SwiGLU epilogue, silu(gate)*up is requantised to e4m3 1x128
// (epilogue fusion, walkthrough sec. 3.2).
//
// gfx950 mapping
//   * v_mfma_f32_16x16x128_f8f6f4: one instruction covers one 16x16 output tile over
//     exactly one 128-deep scale block, so promotion is one fp32 FMA per output per
//     block: acc += (sA*sB) * mfma(b, a, 0).  With the weight fragment as the A operand
//     the partial is the transposed tile, so a lane's four values share one output row
//     (one row scale per step) and are four consecutive columns (wide epilogue stores).
//   * 512 threads = 8 wave64s, two per SIMD: the promotion arithmetic of one wave runs
//     while the other wave's MFMAs occupy the matrix core.  A workgroup tile is BM rows x
//     256 weight rows (plain: 256 output columns; SwiGLU: 128 gate + 128 up rows, so the
//     1x128 requant block is complete in one workgroup).  The waves split the weight rows
//     (32 each) and all share the BM activation rows.  Large groups use BMB = 128 or 192
//     rows per tile (two instances; the launcher picks one per launch): a 192-row tile
//     moves 22% fewer operand bytes per FLOP, and fits the 256 registers a wave has at two
//     waves per SIMD with one fragment step of read-ahead, a two-block weight ring and
//     three activation stages, its epilogue staged in two 96-row passes.
//   * Weights are stored fragment-major (moe_pack_weight_fp8): the 2 KB a wave needs
//     for one 16-row x 128-deep fragment are contiguous, in the order the MFMA takes
//     them, and go straight from memory to registers -- no LDS traffic, fully coalesced
//     loads, three K blocks in flight per wave (two in 192-row tiles, six in small ones).
//   * Activation rows (gathered through a_rows) reach LDS by direct global->LDS DMA into
//     four stages (three in 192-row tiles), in a 16-byte XOR swizzle read back without
//     bank conflicts.  One barrier per K block, placed two fragment steps (192-row
//     tiles: one) before the block ends; the reads of those last steps already fetch the
//     next block's first fragments, so the MFMAs never wait on the barrier.
//   * The tile's activation scales for all K blocks are transposed into LDS once per
//     tile, so that the K loop loads no scattered scale words; for large tiles with
//     K <= 8192 (192-row tiles: K <= 4096) the table holds the products sA*sB (one table
//     per weight-scale block of the tile), so the promotion needs no multiply in the K
//     loop.
//   * Persistent grid; workgroup b works on tiles v, v+P, ... with v = (b mod 8) * P/8 +
//     b/8, so that the 32 tiles one XCD holds at a time are consecutive; inside a group
//     they run down up to 16 row tiles before moving to the next column tile, so those
//     tiles share a few activation row tiles and weight column tiles in that XCD's L2.
//     The tiles of large groups (MFMA-bound) and of small groups (bound by the weight
//     stream) are interleaved by XCD-sized windows in proportion to their counts, so
//     both kinds run at once while each XCD's L2 serves one kind at a time.
#pragma once
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace moe {

namespace gemm_detail {
struct GemmArgs {
  const uint8_t* A;
  const float* sA;
  const int32_t* a_rows;
  int a_row_div;
  const uint8_t* Bf;  // fragment-major weights
  const int32_t* offsets;
  int G;
  int N;  // output columns
  int K;
  void* C;
  float* sC;
  int mode, cap;  // GroupRows of the tile map and its C (masked) or M (dense)
  // W4: the per-row weight scales, read with vector loads.  Deliberately not the
  // restrict kernel argument: a restrict pointer's loads may be moved across the
  // compiler fence that keeps every block's count of vector memory operations in
  // order, which the counted waits for the activation copies rely on.
  const float* wsc;
  // >= 0: a 256-row-tile launch with that many row tiles per round handles the leading
  // whole 256-row tiles (big_cut); this launch takes the rest of every group
  int big_rpr;
};

// wait for this wave's LDS operations, then for the whole workgroup
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
}  // namespace gemm_detail
using gemm_detail::GemmArgs;
using gemm_detail::lds_barrier;

// 4-bit weights as FP8 MFMA operands: the codes -7..7 are exact e4m3 values, so the
// matrix core multiplies them exactly.  One 32-bit word holds 8 consecutive k, byte b
// carrying k = b in its low nibble and k = 4 + b in its high nibble, each nibble sign
// (bit 3) and magnitude (bits 0-2).  A byte permute looks the four magnitudes of a
// nibble half up in the e4m3 codes of 0..7 (0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C,
// 0x4E) and the sign goes to bit 7: the lane's 32 codes, in k order, as the 32 bytes of
// its MFMA operand.
__device__ __forceinline__ v8i expand_int4_e4m3(v4i w) {
  constexpr uint32_t T03 = 0x44403800u, T47 = 0x4E4C4A48u;
  v8i r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t x = (uint32_t)w[p];
    r[2 * p] = (int)(__builtin_amdgcn_perm(T47, T03, x & 0x07070707u) |
                     ((x << 4) & 0x80808080u));
    r[2 * p + 1] = (int)(__builtin_amdgcn_perm(T47, T03, (x >> 4) & 0x07070707u) |
                         (x & 0x80808080u));
  }
  return r;
}

// Two tile classes share one persistent tile list: groups with at most BMS rows get
// BMS-row tiles (their cost is the weight stream), larger groups 128-row tiles.
// The weight scales come as a separate restrict argument: the compiler can then prove
// that no store of the kernel changes them and fetch them with scalar loads (one per
// wave and K block, off the vector memory path).
// W4: the weights are 4-bit codes in [-7, 7] with one fp32 scale per output channel and
// 128-deep K block (expand_int4_e4m3 below), whose scales, packed [G][R/16][K/128][16],
// the kernel reads through args.wsc.  Otherwise e4m3 codes with 128x128 block scales sB.
template <int BMS, bool SWIGLU, bool W4 = false, int BMB = 128>
__global__ __launch_bounds__(512, 1) void gemm_fp8_kernel(GemmArgs args,
                                                           const float* __restrict__ sB) {
  static_assert(BMB == 128 || BMB == 160 || BMB == 192, "large-tile rows");
  constexpr int NW = 8, NT = 512, TN = 2;
  constexpr int BN_OUT = SWIGLU ? 128 : 256;       // output columns per tile
  constexpr int WB = (SWIGLU ? 128 : 256) / NW;    // weight rows per wave (per half: SwiGLU)
  constexpr int A_STAGE = BMB * 128;               // activation codes of one K block
  // activation stage arrays (W4: three, so that its weight ring can be two blocks deep;
  // the ring must cover the activation lead)
  // (192-row tiles: three, for LDS; measured enough at their longer blocks)
  constexpr int NSA = (W4 || BMB > 128) ? 3 : 4;
  // scale table [kb][row], rows of TS floats: the 4-float pad puts the four 16-row
  // groups one fill instruction writes (four consecutive K-block quads) in different banks
  constexpr int TS = BMB + 4;
  constexpr int TAB_FLOATS = (BMB > 128 ? kGemmMaxKBlocks192 : kGemmMaxKBlocks) * TS;
  // epilogue rows of 528 bytes (192-row tiles: staged in two passes of 96 rows)
  constexpr int OUT_FLOATS = (BMB > 128 ? BMB / 2 : BMB) * 132;
  __shared__ TileMap tm;
  // NSA activation stages, each an LDS object of its own (see dma16b; st3 is unused with
  // three); the row-scale table [kb][row] doubles as the epilogue's staging area
  __shared__ __attribute__((aligned(1024))) uint8_t st0[A_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[A_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[A_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[NSA == 4 ? A_STAGE : 16];
  __shared__ __attribute__((aligned(1024))) float tab[TAB_FLOATS > OUT_FLOATS ? TAB_FLOATS : OUT_FLOATS];
  __shared__ int row_src[BMB];
  // product tables: the tile's two weight-scale rows, table t at [t * PT_KB + kb]
  constexpr int PT_KB = TAB_FLOATS / (2 * TS);
  __shared__ float sbt[2 * PT_KB];
  auto stage = [&](auto S) -> uint8_t* {
    constexpr int sidx = decltype(S)::value % NSA;
    if constexpr (sidx == 0) return st0;
    else if constexpr (sidx == 1) return st1;
    else if constexpr (sidx == 2) return st2;
    else return st3;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = args.G, K = args.K, N = args.N, KB = K / 128;
  const int tiles_n = (N + BN_OUT - 1) / BN_OUT;
  const int R = SWIGLU ? 2 * N : N;                // weight rows per group
  const int R16 = R / 16, RB = R / 128;
  const int gsel = 2 * (lane >> 4);
  // 16-byte piece p of LDS row r sits in slot p ^ swz(r).  The LDS has 64 four-byte
  // banks (two 128-byte rows per bank line) and serves a 16-byte read for lanes
  // {0-7, 16-23}, {8-15, 24-31}, {32-39, 48-55}, {40-47, 56-63} together (measured: the
  // bank-conflict counter).  A fragment read gives those 16 lanes rows r..r+7 at pieces
  // 2c ^ swz and (2c + 2) ^ swz; keys taking the values 0, 1, 4, 5 over the four rows
  // of one parity put the 16 reads in 16 different bank groups.
  auto swz = [](int r) {
    const int k = (r >> 1) & 3;
    return (k & 1) | ((k & 2) << 1);
  };

  __shared__ int skip_s[kMaxGroups + 1];
  build_tile_map<BMS, BMB, NT, true>(tm, args.offsets, G, args.mode, args.cap, args.big_rpr,
                                     skip_s);
  // large-group (128-row, MFMA-bound) and small-group (weight-streaming) tile lists
  const int n_big = tm.start[G] * tiles_n, n_small = tm.sstart[G] * tiles_n;
  const int P = gridDim.x, b = blockIdx.x;
  const int v = (P % 8 == 0) ? (b % 8) * (P / 8) + b / 8 : b;

  // PROD (K <= PT_KB blocks): the table holds each row scale already multiplied by the
  // weight scale of the block, one table per 128-column weight block the tile touches
  // (plain: the tile's two halves; SwiGLU: gate and up), so promotion is a bare FMA.
  // The product is rounded once, as the in-loop product of the other form is.
  auto run_tile = [&](auto BMC, auto PRODC, int g, int row0, int row_end, int n0) {
    constexpr int BM = decltype(BMC)::value;
    constexpr bool PROD = decltype(PRODC)::value;
    constexpr int TM = BM / 16;                    // 16-row MFMA tiles per wave
    // weight ring: blocks kb .. kb+DB-1.  Small tiles only stream weights, so they keep
    // more blocks in flight (their accumulators are few).
    // (W4: half the bytes per block and a larger register set per block, so fewer)
    // (192-row tiles: two, for registers)
    constexpr int DB = BM <= 32 ? (W4 ? 4 : 6) : ((W4 || BM > 128) ? 2 : 3);
    constexpr int LEAD = NSA - 1;                  // activation DMA runs LEAD blocks ahead
    static_assert(LEAD <= DB, "prologue order");
    // the K loop is unrolled by UNR blocks, so that weight slots and activation stages
    // are compile-time in every block
    // (and by a multiple of the fragment ring's 3 sets, so every ring phase repeats)
    constexpr int UNR0 = DB * NSA / gcd_c(DB, NSA);
    constexpr int UNR = UNR0 % 3 == 0 ? UNR0 : 3 * UNR0;
    const int n_valid = min(row_end - row0, BM);   // >= 1
    const int ncols = min(BN_OUT, N - n0);         // plain N % 256 == 128: half last tile
    if (tid < BM) {
      // source row of every tile row; rows past the group's end repeat its last row and
      // their results are discarded
      const int lr = min(row0 + tid, row_end - 1);
      int src = lr;
      if (args.a_rows) {
        const int sr = args.a_rows[lr];
        src = sr < 0 ? 0 : sr / args.a_row_div;
      }
      row_src[tid] = src;
    }
    if constexpr (PROD) {
      // weight-scale rows of the tables; plain: the second half's block (clamped for a
      // half last tile, whose second-half waves use the first table)
      const int cb0 = n0 / 128;
      const int cb1 = SWIGLU ? (N + n0) / 128 : min(cb0 + 1, RB - 1);
      // (192-row tiles: the thread index made opaque here, so that these addresses are
      // formed per tile instead of being hoisted out of the tile loop into registers)
      int tq = tid;
      if constexpr (BMB > 128) asm volatile("" : "+v"(tq));
      if (tq < 2 * PT_KB) {
        const int t = tq / PT_KB, kb = tq - t * PT_KB;
        if (kb < KB) sbt[tq] = sB[((size_t)g * RB + (t ? cb1 : cb0)) * KB + kb];
      }
    }
    __syncthreads();

    // ---- activation DMA: an instruction fills 8 rows (1 KB); lane L lands at row L/8,
    // slot L%8 and fetches global piece (L%8) ^ swz(row).  Every wave issues ADMA
    // instructions per block (small tiles repeat row groups, same bytes to same place).
    constexpr int GROUPS = BM / 8;
    constexpr int ADMA = GROUPS > NW ? (GROUPS + NW - 1) / NW : 1;  // (160 rows: 20 groups)
    uint32_t a_voff[ADMA], a_m[ADMA];
#pragma unroll
    for (int q = 0; q < ADMA; ++q) {
      const int grp = (wid + NW * q) % GROUPS;
      const int row = grp * 8 + (lane >> 3), slot = lane & 7;
      a_voff[q] = (uint32_t)row_src[row] * (uint32_t)K + ((slot ^ swz(row)) << 4);
      a_m[q] = grp * 1024;
    }
    // (fenced, like load_b: the counted waits need the issue order kept)
    auto dma_a = [&](auto S, int kb) {
      uint8_t* st = stage(S);
      const uint8_t* base = args.A + (size_t)min(kb, KB - 1) * 128;
#pragma unroll
      for (int q = 0; q < ADMA; ++q) dma16b(base, a_voff[q], st + a_m[q]);
      asm volatile("" ::: "memory");
    };

    // ---- the tile's row scales, transposed into LDS [kb][row].  Item (row, q) holds
    // blocks 4q .. 4q+3 of one row, fetched as one 16-byte load; consecutive lanes take
    // 16 consecutive rows, then the next q, so one wave instruction covers 16 rows x 64
    // contiguous bytes instead of 64 scattered rows.  A thread issues all loads of a
    // round before its LDS writes, so the latency is paid once per round.
    {
      constexpr int TAB_IT = 4;                    // items per thread per round
      constexpr int RSTEP = NT / 16;               // item quads between a thread's items
      const int nq = (KB + 3) / 4;
      const int tab_items = BM * nq;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(args.sA), (short)0, -1, 0x00020000);
      // item p: row group rb = (p / 16) / nq, quad q = (p / 16) % nq, row rb*16 + p%16.
      // A thread's items are RSTEP apart in p / 16: (rb, q) advance by a fixed step.
      const int drb = RSTEP / nq, dq = RSTEP - drb * nq;
      int rb = (tid >> 4) / nq, q = (tid >> 4) - rb * nq;
      const int rlo = tid & 15;
      for (int p0 = 0; p0 < tab_items; p0 += TAB_IT * NT) {
        v4i tv[TAB_IT];
        int rowv[TAB_IT], qv[TAB_IT];
#pragma unroll
        for (int it = 0; it < TAB_IT; ++it) {
          rowv[it] = rb * 16 + rlo;
          qv[it] = q;
          if (p0 + tid + it * NT < tab_items) {
            const uint32_t base = (uint32_t)row_src[rowv[it]] * (uint32_t)KB;
            if (4 * q + 3 < KB) {
              tv[it] = __builtin_bit_cast(
                  v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, (base + 4 * q) * 4u, 0, 0));
            } else {                                 // the row's last, partial chunk
#pragma unroll
              for (int t = 0; t < 4; ++t)
                tv[it][t] = (int)__builtin_amdgcn_raw_buffer_load_b32(
                    rs, (base + (uint32_t)min(4 * q + t, KB - 1)) * 4u, 0, 0);
            }
          }
          rb += drb;
          q += dq;
          if (q >= nq) {
            q -= nq;
            ++rb;
          }
        }
#pragma unroll
        for (int it = 0; it < TAB_IT; ++it) {
          if (p0 + tid + it * NT < tab_items) {
            const int row = rowv[it];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int kb = 4 * qv[it] + t;
              if (kb < KB) {
                const float a = __int_as_float(tv[it][t]);
                if constexpr (PROD) {
                  tab[kb * TS + row] = a * sbt[kb];
                  tab[(PT_KB + kb) * TS + row] = a * sbt[PT_KB + kb];
                } else {
                  tab[kb * TS + row] = a;
                }
              }
            }
          }
        }
      }
    }

    // ---- this wave's weight fragments: a scalar base plus the lane's 16-byte offset.
    // Waves past a half last tile repeat valid rows; their results are not stored.
    const int wcol = WB * wid < ncols ? WB * wid : 0;
    const int brow0 = n0 + wcol;
    constexpr size_t FRAG = W4 ? 1024 : 2048;      // bytes of one 16-row x 128-deep fragment
    const uint8_t* b_base = args.Bf + (((size_t)g * R16 + brow0 / 16) * (size_t)KB) * FRAG;
    const size_t b_step = (size_t)KB * FRAG;       // next 16-row block
    // plain: fragment j is block j; SwiGLU: j = 0 gate, j = 1 the up row N further on
    const size_t b_next = SWIGLU ? (size_t)(N / 16) * b_step : b_step;
    const uint32_t b_lane = lane * 16;
    const float* sb0 = sB + ((size_t)g * RB + brow0 / 128) * KB;
    const float* sb1 = sB + ((size_t)g * RB + (SWIGLU ? (N + brow0) / 128 : 0)) * KB;
    // W4: the scales of the lane's four weight rows 4 (lane / 16) .. +3 of a fragment
    const float* s7_base =
        args.wsc + (((size_t)g * R16 + brow0 / 16) * (size_t)KB) * 16 + 4 * (lane >> 4);
    const size_t s7_next = SWIGLU ? (size_t)(N / 16) * KB * 16 : (size_t)KB * 16;
    constexpr int NB_OPS = 2 * TN;                 // vector loads per load_b

    // The barrier waits count this wave's vector memory operations (vmcnt), so every
    // load_b must issue exactly NB_OPS of them: the compiler barrier at its end stops a
    // clamped block's repeated addresses from being merged with the previous call's, and
    // the never-taken sink after the K loop keeps the loads of blocks past the end alive.
    // W4: the 16 bytes of packed codes per lane and fragment, expanded at the block start
    using BQ = std::conditional_t<W4, v4i, v8i>;
    BQ bq[DB][TN];
    float sbq[DB][2];
    v4f s7q[W4 ? DB : 1][TN];
    auto load_b = [&](int slot, int kb) {
      kb = min(kb, KB - 1);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint8_t* p = b_base + (size_t)j * b_next + (size_t)kb * FRAG;
        if constexpr (W4) {
          bq[slot][j] = *reinterpret_cast<const v4i*>(p + b_lane);
          s7q[slot][j] =
              *reinterpret_cast<const v4f*>(s7_base + (size_t)j * s7_next + (size_t)kb * 16);
        } else {
          // small SwiGLU tiles (the layer's up/gate projection for light experts: pure
          // weight streams over K = d) load non-temporally, which measured 6-8% faster
          // there; in the plain instance (the down projection, K = I) it was slower
          v4i lo, hi;
          if constexpr (BM <= 32 && SWIGLU) {
            lo = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p + b_lane));
            hi = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p + 1024 + b_lane));
          } else {
            lo = *reinterpret_cast<const v4i*>(p + b_lane);
            hi = *reinterpret_cast<const v4i*>(p + 1024 + b_lane);
          }
          bq[slot][j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
      if constexpr (!PROD && !W4) {
        sbq[slot][0] = sb0[kb];
        sbq[slot][1] = SWIGLU ? sb1[kb] : 0.f;
      }
      asm volatile("" ::: "memory");
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    // A fragments and their row scales run RA steps ahead of their MFMAs through rings of
    // AR sets; the reads of a block's last RA steps fetch the next block's first
    // fragments, published by the barrier RA steps before the block ends.  Promotion of
    // a step's partials runs one step behind its MFMAs (rings of PR), across blocks.
    // Ring phases are compile-time because the K loop is unrolled by DB blocks.
    // PROD: a step's promotion reads its scale set straight from the ring (SR sets, one
    // more than the fragments, so the set is still there one step later); otherwise
    // the scale products are formed in the step (cq).
    // (192-row tiles: one step ahead, a ring of two, for registers)
    constexpr int RA = TM < 2 ? TM : (TM > 8 ? 1 : 2);
    constexpr int AR = (RA == 1 && TM > 8) ? 2 : 3;  // divides UNR * TM
    constexpr int SR = (PROD || W4) ? RA + 2 : AR;
    constexpr int PR = (TM % 2 == 0) ? 2 : 3;      // divides UNR * TM
    constexpr int NSC = (PROD && SWIGLU) ? 2 : 1;  // scale sets per step
    static_assert((UNR * TM) % AR == 0 && (UNR * TM) % PR == 0 && (UNR * TM) % SR == 0,
                  "ring phases");
    v8i af[AR];
    float sa[SR][NSC];
    v4f pp[PR][TN];
    float cq[PROD ? 1 : PR][2];
    // plain PROD: the table of this wave's half
    const float* tabw = tab + ((PROD && !SWIGLU && wcol >= 128) ? PT_KB * TS : 0);
    auto rd_a = [&](const uint8_t* L, int i) {
      const int row = i * 16 + (lane & 15);
      const uint8_t* base = L + row * 128;
      const v4i lo = *reinterpret_cast<const v4i*>(base + ((gsel ^ swz(row)) << 4));
      const v4i hi = *reinterpret_cast<const v4i*>(base + (((gsel + 1) ^ swz(row)) << 4));
      return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    // the scale of this lane's output row (see the MFMA operand order below)
    auto rd_s = [&](int kbx, int i, int t = 0) {
      return tabw[(t * PT_KB + kbx) * TS + i * 16 + (lane & 15)];
    };
    auto rd_sets = [&](int sslot, int kbx, int i) {
#pragma unroll
      for (int t = 0; t < NSC; ++t) sa[sslot][t] = rd_s(kbx, i, t);
    };
    // W4: promote with the row scale and each output column's own weight scale (the
    // scales of the block the partials belong to: weight-ring slot wslot)
    auto promote_w4 = [&](int slot, int sslot, int ii, int wslot) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[ii][j][r] =
              fmaf(pp[slot][j][r] * s7q[wslot][j][r], sa[sslot][0], acc[ii][j][r]);
    };
    // promote the partials in pp[slot] (scales: ring set sslot, PROD) into row tile ii
    auto promote = [&](int slot, int sslot, int ii) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int h = (SWIGLU && j >= TN / 2) ? 1 : 0;
        float c;
        if constexpr (PROD) c = sa[sslot][NSC > 1 ? h : 0];
        else c = cq[slot][h];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[ii][j][r] = fmaf(c, pp[slot][j][r], acc[ii][j][r]);
      }
    };

    // one K block.  Vector memory order per block: weights of block kb+DB-1, then the
    // activation DMA of block kb+3 into the stage block kb-1 used (every wave finished
    // that stage before the previous block's barrier).
    auto body = [&](auto U, int kb) {
      constexpr int u = decltype(U)::value;
      constexpr int ub = u % DB;
      constexpr int g0 = u * TM;                   // step index within the unrolled round
      // the activation DMA goes out mid-block where that is still before the barrier
      // step (128-row tiles: spreads the block's vector memory issue, ~1% faster); the
      // barrier's wait count is the same either way
      constexpr int DMA_STEP = (TM / 2 < TM - RA) ? TM / 2 : 0;
      if constexpr (W4) {
        // the previous block's last step, before its weight-ring slot (and scales) is
        // reloaded just below
        if (kb > 0)
          promote_w4((g0 + UNR * TM - 1) % PR, (g0 + UNR * TM - 1) % SR, TM - 1,
                     (u + DB - 1) % DB);
      }
      load_b((u + DB - 1) % DB, kb + DB - 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (DMA_STEP == 0) {
        dma_a(std::integral_constant<int, u + LEAD>{}, kb + LEAD);
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint8_t* L = stage(U);
      const uint8_t* Ln = stage(std::integral_constant<int, u + 1>{});
      [[maybe_unused]] const float sbA = W4 ? 0.f : sbq[ub][0];
      [[maybe_unused]] const float sbB = W4 ? 0.f : (SWIGLU ? sbq[ub][1] : sbq[ub][0]);
      // W4: this block's weights as e4m3 codes
      [[maybe_unused]] v8i bx[W4 ? TN : 1];
      if constexpr (W4) {
#pragma unroll
        for (int j = 0; j < TN; ++j) bx[j] = expand_int4_e4m3(bq[ub][j]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int gs = g0 + i;
        if (DMA_STEP > 0 && i == DMA_STEP) {
          __builtin_amdgcn_sched_barrier(0);
          dma_a(std::integral_constant<int, u + LEAD>{}, kb + LEAD);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (i == TM - RA) {
          // this wave's DMA of block kb+1 (issued two blocks ago) has landed: after it
          // came the two later blocks' weight loads and DMAs.  The barrier publishes
          // block kb+1; every wave's reads of stage kb%NSA before it are done.
          wait_vmcnt<(LEAD - 1) * (NB_OPS + ADMA)>();
          lds_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
        {
          const int ni = i + RA;
          const int slot = (gs + RA) % AR, sslot = (gs + RA) % SR;
          if (ni < TM) {
            af[slot] = rd_a(L, ni);
            rd_sets(sslot, kb, ni);
          } else {
            af[slot] = rd_a(Ln, ni - TM);
            rd_sets(sslot, min(kb + 1, KB - 1), ni - TM);
          }
        }
        // weights as the A operand, activations as B: the 16x16 partial is the transposed
        // tile, each lane holding four consecutive output columns of one output row
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          v8i wop;
          if constexpr (W4) wop = bx[j];
          else wop = bq[ub][j];
          pp[gs % PR][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wop, af[gs % AR], zero, 0, 0, 0, 0, 0, 0);
        }
        if constexpr (!PROD && !W4) {
          cq[gs % PR][0] = sa[gs % SR][0] * sbA;
          cq[gs % PR][1] = sa[gs % SR][0] * sbB;
        }
        // the previous step's partials (before the tile's first block: zeros)
        if constexpr (W4) {
          if (i > 0) promote_w4((gs + UNR * TM - 1) % PR, (gs + UNR * TM - 1) % SR, i - 1, ub);
        } else
          promote((gs + UNR * TM - 1) % PR, (gs + UNR * TM - 1) % SR, i > 0 ? i - 1 : TM - 1);
        // issue order inside a step: MFMA, the next fragment's two reads, four promotion
        // FMAs, MFMA, the scale read(s), four FMAs (the reads between the MFMAs measured
        // 1-2% faster than all reads first); nothing moves across steps
        static_assert(TN == 2, "step schedule");
        constexpr int VPS = W4 ? 8 : 4;             // promotion VALU per half step
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, VPS, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NSC, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, VPS, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // prologue: block 0's activations in LDS, the weights of blocks 0 .. DB-2 and the
    // activations of blocks 1 and 2 in flight, the first RA fragments of block 0 in
    // registers (block kb issues the weights of kb+DB-1, then the activations of kb+3:
    // replayed for the blocks before 0, so the vector memory order is the steady one)
    constexpr int KPRE = DB - 1 > LEAD ? DB - 1 : LEAD;
    // Every copy is fenced: the wait below counts operations in issue order, and without
    // the fences the compiler may move a later block's weight loads above an earlier
    // activation copy (seen where the weight ring is shallower than the activation lead,
    // so the first replayed block has no weight loads to fence it).
    static_for<KPRE>([&](auto T) {
      constexpr int k = KPRE - decltype(T)::value;   // "block -k"
      if constexpr (DB - 1 - k >= 0) load_b(DB - 1 - k, DB - 1 - k);
      if constexpr (LEAD - k >= 0) {
        dma_a(std::integral_constant<int, LEAD - k>{}, LEAD - k);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
    wait_vmcnt<(LEAD - 1) * (NB_OPS + ADMA)>();
    lds_barrier();
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      af[i] = rd_a(stage(std::integral_constant<int, 0>{}), i);
      rd_sets(i, 0, i);
    }
    // the first step promotes zeros: partials and scales of the sets not yet read
#pragma unroll
    for (int i = RA; i < SR; ++i)
#pragma unroll
      for (int t = 0; t < NSC; ++t) sa[i][t] = 0.f;
#pragma unroll
    for (int p = 0; p < (PROD ? 1 : PR); ++p) {
      cq[p][0] = 0.f;
      cq[p][1] = 0.f;
    }
#pragma unroll
    for (int p = 0; p < PR; ++p)
#pragma unroll
      for (int j = 0; j < TN; ++j) pp[p][j] = zero;

    int kb = 0;
    for (; kb + UNR <= KB; kb += UNR)
      static_for<UNR>([&](auto U) { body(U, kb + decltype(U)::value); });
    static_for<UNR - 1>([&](auto U) {
      if (kb + decltype(U)::value < KB) body(U, kb + decltype(U)::value);
    });
    if (G < 0) {
      // never taken (G >= 1): uses every weight-ring slot, see load_b
      int x = 0;
#pragma unroll
      for (int d = 0; d < DB; ++d) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
          for (int e = 0; e < (W4 ? 4 : 8); ++e) x ^= bq[d][j][e];
          if constexpr (W4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) x ^= __float_as_int(s7q[d][j][e]);
          }
        }
        if constexpr (!PROD && !W4) x ^= __float_as_int(sbq[d][0]) ^ __float_as_int(sbq[d][1]);
      }
      static_cast<int*>(args.C)[tid] = x;
    }
    {
      // the last block's last step
      const int glast = ((KB - 1) % UNR) * TM + TM - 1;
      static_for<PR>([&](auto P_) {
        static_for<SR>([&](auto S_) {
          constexpr int pv = decltype(P_)::value, sv = decltype(S_)::value;
          if (glast % PR == pv && glast % SR == sv) {
            if constexpr (W4) {
              static_for<DB>([&](auto D_) {
                constexpr int dv = decltype(D_)::value;
                if ((KB - 1) % DB == dv) promote_w4(pv, sv, TM - 1, dv);
              });
            } else {
              promote(pv, sv, TM - 1);
            }
          }
        });
      });
    }
    wait_vmcnt<0>();  // the last (clamped) activation DMAs land before LDS is reused
    lds_barrier();

    // ---- epilogue.  acc[i][j] of a lane: tile row i*16 + lane%16, columns
    // j*16 + 4*(lane/16) + r of the wave's slice (the transposed MFMA tile).
    if constexpr (!SWIGLU) {
      // bf16 tile staged through LDS for 16-byte stores; rows of 528 bytes put the 16
      // rows of one 8-byte write in different banks
      constexpr int OB = 528;
      // passes of RP rows (192-row tiles: two, so the staging fits the table's LDS)
      constexpr int NPASS = BM > 128 ? 2 : 1, RP = BM / NPASS, TMP = TM / NPASS;
      uint8_t* ot = reinterpret_cast<uint8_t*>(tab);
      uint8_t* C = static_cast<uint8_t*>(args.C);
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) {
#pragma unroll
        for (int ii = 0; ii < TMP; ++ii) {
          const int i = ps * TMP + ii;
          const int trow = ii * 16 + (lane & 15);
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int tcol = wid * WB + j * 16 + (lane >> 4) * 4;
            const uint32_t lo = (uint32_t)f32_to_bf16(acc[i][j][0]) |
                                ((uint32_t)f32_to_bf16(acc[i][j][1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(acc[i][j][2]) |
                                ((uint32_t)f32_to_bf16(acc[i][j][3]) << 16);
            *reinterpret_cast<uint2*>(ot + trow * OB + tcol * 2) = make_uint2(lo, hi);
          }
        }
        __syncthreads();
        if (ncols == BN_OUT) {
          // full tile: thread tid takes 16-byte chunk tid % 32 of rows tid / 32 + 16 k; all
          // LDS reads go out before the stores
          constexpr int CPR = BN_OUT * 2 / 16, RPP = NT / CPR;
          static_assert(RP % RPP == 0, "store passes");
          const int ch = tid % CPR, tr0 = tid / CPR;
          v4i ov[RP / RPP];
#pragma unroll
          for (int k = 0; k < RP / RPP; ++k)
            ov[k] = *reinterpret_cast<const v4i*>(ot + (tr0 + k * RPP) * OB + ch * 16);
#pragma unroll
          for (int k = 0; k < RP / RPP; ++k) {
            const int trow = ps * RP + tr0 + k * RPP;
            if (trow < n_valid)
              *reinterpret_cast<v4i*>(C + ((size_t)(row0 + trow) * N + n0) * 2 + ch * 16) = ov[k];
          }
        } else {
          const int cpr = ncols * 2 / 16;            // 16-byte chunks per valid row
          const int nv = min(n_valid - ps * RP, RP);
          for (int c = tid; c < nv * cpr; c += NT) {
            const int trow = c / cpr, ch = c % cpr;
            *reinterpret_cast<v4i*>(C + ((size_t)(row0 + ps * RP + trow) * N + n0) * 2 +
                                    ch * 16) =
                *reinterpret_cast<const v4i*>(ot + trow * OB + ch * 16);
          }
        }
        if (NPASS > 1) __syncthreads();
      }
    } else {
      // h = silu(gate) * up goes to LDS in fp32 (row stride 132 floats); then four
      // threads per row take the row's 1x128 block: max |h|, the scale, the codes
      constexpr int HS = 132;
      constexpr int NPASS = BM > 128 ? 2 : 1, RP = BM / NPASS, TMP = TM / NPASS;
      float* hsm = tab;
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) {
#pragma unroll
        for (int ii = 0; ii < TMP; ++ii) {
          const int i = ps * TMP + ii;
          const int trow = ii * 16 + (lane & 15);
          const int tcol = wid * WB + (lane >> 4) * 4;
          v4f h;
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = silu_fast(acc[i][0][r]) * acc[i][1][r];
          *reinterpret_cast<v4f*>(hsm + trow * HS + tcol) = h;
        }
        __syncthreads();
        const int row = tid >> 2, part = tid & 3;
        float hv[32];
        float m = 0.f;
        if (row < RP) {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const v4f x = *reinterpret_cast<const v4f*>(hsm + row * HS + part * 32 + q * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              hv[q * 4 + e] = x[e];
              m = fmaxf(m, fabsf(x[e]));
            }
          }
        }
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        const int grow = ps * RP + row;
        if (row < RP && grow < n_valid) {
          // the activation quantiser's rule: s = fl32(amax / 448), q = e4m3(fl32(h / s)),
          // with correctly rounded divisions (not a multiply by a rounded reciprocal)
          const float sc = block_scale(m);
          uint32_t w[8];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            w[q] = e4m3x4(clamp448(hv[4 * q] / sc), clamp448(hv[4 * q + 1] / sc),
                          clamp448(hv[4 * q + 2] / sc), clamp448(hv[4 * q + 3] / sc));
          uint8_t* C =
              static_cast<uint8_t*>(args.C) + (size_t)(row0 + grow) * N + n0 + part * 32;
          *reinterpret_cast<v4i*>(C) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
          *reinterpret_cast<v4i*>(C + 16) = v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
          if (part == 0) args.sC[(size_t)(row0 + grow) * (N / 128) + n0 / 128] = sc;
        }
        if (NPASS > 1) __syncthreads();
      }
    }
    __syncthreads();  // LDS (row_src, table, stages) is reused by the next tile
  };

  // The two lists are interleaved in windows of Q = P/8 consecutive tiles, the tiles
  // one XCD holds at a time: a window is all large-group or all small-group tiles, and
  // windows of the two kinds alternate in proportion to their counts.  So every XCD's
  // L2 serves one kind at a time (mixing them per tile evicts the reused activation and
  // weight tiles: 25% more fabric traffic), while the machine runs both at once.
  const int Q = (P % 8 == 0) ? P / 8 : 1;
  const int nbq = (n_big + Q - 1) / Q, nsq = (n_small + Q - 1) / Q, nq = nbq + nsq;
  for (int t = v; t < nq * Q; t += P) {
    // ---- locate the tile: within a group, runs of up to GM row tiles are walked column
    // tile by column tile
    constexpr int GM = 16;
    // window tb holds large-group tiles if floor(tb nbq / nq) steps at tb; slots past
    // the end of a list hold no tile
    const int tb = t / Q, to = t - tb * Q;
    const int b0 = (int)((long long)tb * nbq / nq);
    const int b1 = (int)((long long)(tb + 1) * nbq / nq);
    const bool big = b1 > b0;
    const int j = (big ? b0 : tb - b0) * Q + to;
    if (j >= (big ? n_big : n_small)) continue;
    const int* st = big ? tm.start : tm.sstart;
    const int g = find_group(st, G, j, tiles_n);
    const int mt = st[g + 1] - st[g];
    const int local = j - st[g] * tiles_n;
    const int sr = local / (GM * tiles_n);
    const int rows_sr = min(GM, mt - sr * GM);
    const int idx = local - sr * GM * tiles_n;
    const int mi = sr * GM + idx % rows_sr, ni = idx / rows_sr;
    // tile coordinates are the same in every lane: scalar registers
    const int gu = __builtin_amdgcn_readfirstlane(g);
    const int* skip = args.big_rpr >= 0 ? skip_s : nullptr;
    const int rows = __builtin_amdgcn_readfirstlane(group_rows(tm, gu, skip));
    const int r0 = __builtin_amdgcn_readfirstlane(group_row0(tm, gu, skip));
    const int n0 = __builtin_amdgcn_readfirstlane(ni * BN_OUT);
    const int miu = __builtin_amdgcn_readfirstlane(mi);
    // small tiles stream weights and gain nothing from the product tables (their
    // VALU work hides behind the loads), so only 128-row tiles use them
    using P1 = std::integral_constant<bool, true>;
    using P0 = std::integral_constant<bool, false>;
    if (rows <= BMS)
      run_tile(std::integral_constant<int, BMS>{}, P0{}, gu, r0 + miu * BMS, r0 + rows, n0);
    else if (!W4 && KB <= PT_KB)
      run_tile(std::integral_constant<int, BMB>{}, P1{}, gu, r0 + miu * BMB, r0 + rows, n0);
    else
      run_tile(std::integral_constant<int, BMB>{}, P0{}, gu, r0 + miu * BMB, r0 + rows, n0);
  }
}

// Grid and template instance of one grouped GEMM launch (the instances a launcher
// uses are compiled in its own source file).  bmb: rows of the large-group tiles, 128 or
// (K <= 128 * kGemmMaxKBlocks192) 192, or (4-bit weights) 160.
template <bool W4>
hipError_t launch_gemm_impl(const uint8_t* A, const float* sA, const int32_t* a_rows,
                            int a_row_div, const uint8_t* Bf, const float* sB,
                            const int32_t* offsets, int G, int R_cap, int N, int K, bool swiglu,
                            void* C, float* sC, int bm, int num_cus, hipStream_t s,
                            int rows_mode, int cap, int big_rpr = -1, int bmb = 128) {
  if (K / 128 > kGemmMaxKBlocks) return hipErrorInvalidValue;
  if (bmb != 128 && ((bmb != 192 && (bmb != 160 || !W4)) || K / 128 > kGemmMaxKBlocks192))
    return hipErrorInvalidValue;
  GemmArgs a{A, sA, a_rows, a_row_div, Bf, offsets, G, N, K, C, sC, rows_mode, cap,
             W4 ? sB : nullptr, big_rpr};
  const long tiles_n = swiglu ? N / 128 : (N + 255) / 256;
  const long mtiles = R_cap / (bm < 128 ? bm : 64) + G;
  long grid = std::min<long>(mtiles * tiles_n, (long)num_cus);
  if (grid >= 8) grid = grid / 8 * 8;
  if (grid < 1) grid = 1;
  dim3 gd((unsigned)grid), bd(512);
  // bm: tile rows of small groups (16, 32 or 64); larger groups use bmb-row tiles.  The
  // 4-bit path has no 64-row instance (its register budget); 64 means 32 there.  192-row
  // tiles pair with 16- and 32-row small tiles only (with 64 the instance spills), so
  // bm = 64 keeps 128-row tiles.
  const int bms = bm >= 64 ? (W4 ? 32 : 64) : bm;
#define MOE_GEMM_CASE(BMSV, SW)                                                            \
  do {                                                                                     \
    if constexpr (BMSV <= 32) {                                                            \
      if (bmb == 192) {                                                                    \
        hipLaunchKernelGGL((gemm_fp8_kernel<BMSV, SW, W4, 192>), gd, bd, 0, s, a, sB);     \
        break;                                                                             \
      }                                                                                    \
      if constexpr (W4) {                                                                  \
        if (bmb == 160) {                                                                  \
          hipLaunchKernelGGL((gemm_fp8_kernel<BMSV, SW, W4, 160>), gd, bd, 0, s, a, sB);   \
          break;                                                                           \
        }                                                                                  \
      }                                                                                    \
    }                                                                                      \
    hipLaunchKernelGGL((gemm_fp8_kernel<BMSV, SW, W4, 128>), gd, bd, 0, s, a, sB);         \
  } while (0)
  if (swiglu) {
    switch (bms) {
      case 16: MOE_GEMM_CASE(16, true); break;
      case 32: MOE_GEMM_CASE(32, true); break;
      case 64:
        if constexpr (!W4) MOE_GEMM_CASE(64, true);
        break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (bms) {
      case 16: MOE_GEMM_CASE(16, false); break;
      case 32: MOE_GEMM_CASE(32, false); break;
      case 64:
        if constexpr (!W4) MOE_GEMM_CASE(64, false);
        break;
      default: return hipErrorInvalidValue;
    }
  }
#undef MOE_GEMM_CASE
  return hipGetLastError();
}

}  // namespace moe
