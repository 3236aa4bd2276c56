/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE FFN layer forward library.
 *
 * The library computes the forward pass of one Mixture-of-Experts FFN layer on
 * one GPU's batch of tokens:
 *   route (biased fp32 softmax top-k, or hash)  ->  dispatch into expert-contiguous
 *   rows  ->  1x128 e4m3 activation quantisation  ->  grouped FP8 GEMM with 128x128
 *   block-scaled weights, fused SwiGLU and requantisation  ->  grouped FP8 down
 *   projection  ->  weighted combine,
 * as the MegaMoE/DeepGEMM walkthrough (discosf.com) describes it in sec. 2.1-2.2
 * (layer maths) and sec. 3.2-3.3 (grouped GEMM and FP8), with the hash routing
 * and 4-bit block weights of the DeepSeek-V4 lecture (tqpw.cn, sec. 2.2 and 3.1).
 *
 * Conventions shared by every call
 *   - Every pointer is a DEVICE pointer owned by the caller (host-side scalars are
 *     passed by value).  The library allocates no device memory, keeps no pointer
 *     after it returns and never synchronises the host: each call only enqueues
 *     kernels on `stream` (a hipStream_t passed as void*; NULL = the null stream).
 *   - Row-major layouts.  GEMM operands are K-contiguous ("NT"): A is [rows, K],
 *     B is [G, N, K]; K, and the hidden and intermediate sizes, are multiples of 128.
 *   - Arguments are checked before anything is launched; a bad argument returns a
 *     negative moe_status and leaves every buffer untouched.  A device that is not
 *     gfx950 gives MOE_ERR_UNSUPPORTED (the analogue of the walkthrough's "FP8 not
 *     supported on this GPU", sec. 5.1).  A failed launch gives MOE_ERR_HIP.  Device
 *     faults surface at the caller's next synchronisation.  moe_last_error() holds a
 *     thread-local message for the last non-OK status.
 *   - Outputs are fully overwritten (no accumulate mode).  Identical inputs give
 *     bitwise identical outputs: no floating-point atomics are used.
 *   - Calls on different streams may run concurrently; calls on one stream are
 *     ordered by the stream.
 *   - A call checks and launches on the current HIP device: `stream` and every
 *     pointer must belong to that device.
 */
#ifndef FP8GG_MOE_H
#define FP8GG_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* bad shape, dtype, flag or null pointer */
  MOE_ERR_UNSUPPORTED = -2,  /* current device is not gfx950 / no device */
  MOE_ERR_HIP = -3,          /* a HIP runtime call or kernel launch failed */
  MOE_ERR_WORKSPACE = -4     /* workspace smaller than moe_layer_workspace_size() */
} moe_status;

typedef enum {
  MOE_F32 = 0,   /* IEEE fp32 */
  MOE_BF16 = 1,  /* bfloat16 stored as uint16 */
  MOE_E4M3 = 2,  /* OCP e4m3 ("fn": max 448, no infinities) stored as uint8 */
  MOE_INT4 = 3   /* signed 4-bit codes in [-7, 7], sign-magnitude nibbles, two per byte:
                    byte 4p+b holds code 8p+b (low nibble) and 8p+4+b (high nibble) */
} moe_dtype;

/* moe_route flags */
#define MOE_ROUTE_RENORM 1u  /* divide the k gate weights by their sum */

/* grouped GEMM epilogues */
#define MOE_EPI_PLAIN 0       /* C = A.B^T written in the output dtype of the call   */
#define MOE_EPI_SWIGLU 1      /* B holds 2N rows: [0,N) gate, [N,2N) up;              */
                              /* C = silu(A.Bg^T) * (A.Bu^T), N columns              */

/* layer modes */
#define MOE_MODE_FP32 0   /* fp32 activations and weights, no quantisation            */
#define MOE_MODE_FP8 1    /* e4m3 weights with 128x128 scales, 1x128 activation quant */
#define MOE_MODE_W4A16 2  /* int4 weights with 1x128 per-channel scales, bf16 acts    */
#define MOE_MODE_W4A8 3   /* int4 weights, 1x128 per-channel scales, on the FP8 MFMA  */
                          /* with 1x128 e4m3 activations (moe_pack_weight_int4)     */
#define MOE_LAYOUT_CONTIGUOUS 0 /* expert rows concatenated, each padded to m_align   */
#define MOE_LAYOUT_MASKED 1     /* fixed capacity: expert e owns rows [e C, e C + C)    */
#define MOE_ROUTE_SCORE 0 /* biased softmax top-k over router logits                  */
#define MOE_ROUTE_HASH 1  /* expert = ((id * 2654435761) mod 2^32) mod E, weight 1, k=1 */

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *moe_last_error(void);

/* MOE_OK when HIP device `hip_device` is a gfx950 (MI355X-class) GPU. */
int moe_device_supported(int hip_device);

/* Expert capacity floor(ceil(T*k/E) * factor); 0 when factor <= 0 (dropless).
 * Reproduces ceil(T*k/E)*2 (DeepSeek MoE architecture, mooersco.com, ch. 1) and the
 * worked value 76 for T=2048, k=2, E=64, factor 1.2 (same page, sec. 2.5).
 * Host-only, pure.  Returns a negative moe_status on bad arguments. */
int moe_capacity(int T, int k, int E, double factor);

/* Rows an expert-contiguous buffer may need: T*k + E*(m_align-1).  Host-only. */
size_t moe_rows_bound(int T, int k, int E, int m_align);

/* Router: logits = x . w_router^T, then the biased softmax top-k of
 * moe_route_from_logits.  s_i = softmax(W_g x + b_i) (MegaMoE walkthrough, discosf.com,
 * sec. 2.2); the softmax runs in fp32 (DeepSeek-V4 lecture, tqpw.cn, sec. 2.3).
 *   x [T, d] and w_router [E, d] of dtype x_dt (MOE_BF16 or MOE_F32, both the same);
 *   bias [E] fp32; logits [T, E] fp32 output (always written);
 *   topk_idx [T, k] int32 and topk_w [T, k] fp32 outputs;
 *   ws / ws_bytes: optional device workspace for split-K partial logits; with at least
 *   moe_route_workspace_size() bytes the logit product is split along d over more
 *   workgroups, whose partial sums are added in a fixed order (deterministic for a
 *   given shape; the split changes the fp32 summation order, so logits with and
 *   without a workspace may differ in their last bits); NULL or smaller runs unsplit.
 *   1 <= k <= min(E, 64), E <= 1024; d a multiple of 128 for MOE_BF16. */
int moe_route(const void *x, moe_dtype x_dt, const void *w_router, const float *bias,
              int T, int d, int E, int k, unsigned flags, float *logits,
              int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes moe_route uses to split the logit product (0: it never splits). */
size_t moe_route_workspace_size(int T, int d, int E, moe_dtype x_dt);

/* moe_route for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation
 * and the same outputs, bit for bit, as moe_route given a workspace of
 * moe_route_workspace_size() bytes, but the split-K partial logits go to a static
 * device scratch of 32 MiB that the library holds on each GPU it runs on until the
 * process ends.  The call allocates nothing.  Shapes whose partial logits exceed the
 * scratch (moe_route_workspace_size(T, d, E, x_dt) > 32 MiB) are rejected with
 * MOE_ERR_INVALID_ARG before any launch.  Every call on one GPU shares that scratch:
 * calls that overlap on one GPU (different streams, no ordering between them) race and
 * must not be issued.  Arguments otherwise as moe_route. */
int moe_route_noalloc(const void *x, moe_dtype x_dt, const void *w_router, const float *bias,
                      int T, int d, int E, int k, unsigned flags, float *logits,
                      int32_t *topk_idx, float *topk_w, void *stream);

/* Top-k of fp32 logits [T, E] with per-expert bias [E] (bias may be NULL = 0): the
 * selection and gate weights of s_i = softmax(W_g x + b_i) (MegaMoE walkthrough,
 * discosf.com, sec. 2.1-2.2; fp32 softmax, DeepSeek-V4 lecture, tqpw.cn, sec. 2.3;
 * the renormalised variant is the top-k-then-softmax code of DeepSeek MoE
 * architecture, mooersco.com, ch. 1).  key_e = fl32(logit_e + b_e); the k largest
 * keys are chosen, largest first, equal keys to the lower expert index; topk_w[t, j] = softmax over all E keys at
 * topk_idx[t, j] (or, with MOE_ROUTE_RENORM, divided by the sum of the k chosen).
 * Logits must be finite.  1 <= k <= min(E, 64), E <= 1024. */
int moe_route_from_logits(const float *logits, const float *bias, int T, int E, int k,
                          unsigned flags, int32_t *topk_idx, float *topk_w, void *stream);

/* Hash routing (tqpw.cn sec. 2.2): topk_idx[t] = ((id_t * 2654435761) mod 2^32) mod E,
 * topk_w[t] = 1; k = 1.  token_ids [T] int64 (non-negative); E >= 1. */
int moe_route_hash(const int64_t *token_ids, int T, int E, int32_t *topk_idx,
                   float *topk_w, void *stream);

/* Dispatch of routed slots into expert-contiguous rows (expert grouping,
 * discosf.com sec. 2.1; capacity drop, mooersco.com sec. 2.5).  Slot s = t*k + j.
 *   counts [E]        slots routed to each expert (before capacity)
 *   offsets [E+1]     offsets[0] = 0, offsets[e+1] = offsets[e] + roundup(kept_e, m_align),
 *                     kept_e = min(counts[e], capacity) (counts[e] when capacity = 0)
 *   row_of_slot [T*k] row of each slot, -1 if dropped; within an expert rows follow
 *                     slot order (stable)
 *   slot_of_row [moe_rows_bound(T,k,E,m_align)]  inverse map, -1 on padding rows and
 *                     on every row >= offsets[E]
 * topk_idx [T, k] int32 in [0, E) (with E <= 512 a slot outside that range is dropped:
 * row_of_slot -1, not counted).  1 <= m_align <= 1024; capacity >= 0 (0 = dropless).
 * Integer-only and deterministic. */
int moe_dispatch(const int32_t *topk_idx, int T, int k, int E, int m_align, int capacity,
                 int32_t *counts, int32_t *offsets, int32_t *row_of_slot,
                 int32_t *slot_of_row, void *stream);

/* Dispatch into the fixed-capacity ("masked") expert layout, the second grouped layout
 * DeepGEMM offers beside the contiguous one (qidao123.com day 3), with the capacity of
 * DeepSeek MoE architecture, mooersco.com sec. 2.5: expert e owns rows [e*C, e*C + C)
 * whatever its count; its first min(counts[e], C) slots in slot order take rows e*C,
 * e*C + 1, ... and the rest are dropped silently.  C = capacity (>= 1, e.g. from
 * moe_capacity).  Slot s = t*k + j.
 *   counts [E]          slots routed to each expert (before capacity; the masked GEMM
 *                       clamps them to C)
 *   row_of_slot [T*k]   row of each slot, -1 if dropped
 *   slot_of_row [E*C]   inverse map, -1 on rows no slot took
 * topk_idx [T, k] int32 in [0, E) (with E <= 512 a slot outside that range is dropped).
 * Integer-only and deterministic; the same ranks as moe_dispatch with this capacity. */
int moe_dispatch_masked(const int32_t *topk_idx, int T, int k, int E, int capacity,
                        int32_t *counts, int32_t *row_of_slot, int32_t *slot_of_row,
                        void *stream);

/* 1x128 e4m3 activation quantisation (discosf.com sec. 3.3; fine-grained scales,
 * qidao123.com day 3).  For output row r, source row i = src_row ? src_row[r] / src_div
 * : r (src_row[r] < 0 gives an all-zero row with scale 1); for each 128-wide block:
 * s = fl32(amax / 448) (1 if amax = 0), q = e4m3_rne(clamp(fl32(x / s), -448, 448)).
 *   x [rows_in, K] of dtype x_dt (MOE_BF16 or MOE_F32); q [rows_out, K] uint8;
 *   scales [rows_out, K/128] fp32.  K a multiple of 128; src_div >= 1. */
int moe_quant_fp8(const void *x, moe_dtype x_dt, int rows_in, int K, const int32_t *src_row,
                  int src_div, int rows_out, uint8_t *q, float *scales, void *stream);

/* 128x128 block e4m3 weight quantisation with the same rule, one scale per block:
 * w [G, N, K] fp32 -> q [G, N, K] uint8, scales [G, N/128, K/128] fp32.
 * N and K multiples of 128. */
int moe_quant_weight_fp8(const float *w, int G, int N, int K, uint8_t *q, float *scales,
                         void *stream);

/* Rearranges e4m3 weight codes q [G, N, K] (as moe_quant_weight_fp8 writes them) into
 * the fragment-major layout the FP8 GEMMs read: qf is [G][N/16][K/128][2][64][16 B],
 * where half h, lane l of 16-row block nb and 128-deep block kb hold the 16 codes
 * q[g][16 nb + (l mod 16)][128 kb + 32 (l div 16) + 16 h .. +16] -- the operand of one
 * 16x16x128 matrix instruction in the order a wave loads it.  A pure permutation (same
 * byte count, scales unchanged), done once per weight; q and qf must not overlap.
 * N and K multiples of 128.  (Layout of this library, not of the pages.) */
int moe_pack_weight_fp8(const uint8_t *q, int G, int N, int K, uint8_t *qf, void *stream);

/* Block-wise int4 weights with 1x128 per-channel blocks (tqpw.cn sec. 3.1): for each
 * row n and 128-wide block, scale = max|w| (1 if 0), q = rne(fl32(fl32(w/scale)*7))
 * in [-7,7], s7 = fl32(scale/7).  w [G, N, K] fp32 -> q [G, N, K/2] packed as
 * MOE_INT4 describes, s7 [G, N, K/128] fp32.  K a multiple of 128. */
int moe_quant_weight_int4(const float *w, int G, int N, int K, uint8_t *q, float *s7,
                          void *stream);

/* Grouped FP8 GEMM (discosf.com sec. 3.2: groups differ in M, share N and K; two-level
 * accumulation with fine-grained scales, qidao123.com day 3).  Group g owns logical
 * rows [offsets[g], offsets[g+1]) (offsets on the device, non-decreasing, offsets[0]=0,
 * offsets[G] <= R_cap).  Logical row r reads A row a = a_rows ? a_rows[r] / a_row_div
 * : r (a_rows[r] < 0: any row, output unspecified).  For each 128-deep K block kb
 * the e4m3 products are summed in fp32 and promoted as
 *   acc += sA[a, kb] * sB[g, n/128, kb] * partial.
 *   A [*, K] e4m3, sA [*, K/128] fp32; B: the e4m3 codes of [G, Nb, K] weights in the
 *   fragment-major layout of moe_pack_weight_fp8, sB [G, Nb/128, K/128] fp32, with
 *   Nb = N (MOE_EPI_PLAIN) or 2N (MOE_EPI_SWIGLU).
 *   out_dt MOE_BF16: C [R_cap, N] bf16 (RNE), sC unused;
 *   out_dt MOE_E4M3 (SwiGLU only): C [R_cap, N] e4m3 codes of the fp32 SwiGLU output
 *     quantised 1x128 as moe_quant_fp8, sC [R_cap, N/128] fp32.
 * Rows >= offsets[G] and padding rows are unspecified.  N and K multiples of 128,
 * K <= 16384 (the kernel keeps a tile's activation scales for all K blocks on chip).
 * A is read with 32-bit byte offsets: every A row the call reads must end within the
 * first 2^32 - 256 bytes of A (checked as R_cap * K when a_rows is NULL; with a_rows
 * the caller guarantees it for the rows a_rows names).
 * C and sC must not overlap sB (checked: the kernel reads sB through the scalar cache)
 * nor any other input (not checked).
 * Kernel choice: with FP8GG_BIG_TILES=1 in the environment (read at each call), groups
 * that average at least 256 rows (R_cap / G here, cap for the masked form, M for
 * gemm_fp8, the layer's row bound per expert in moe_layer_fwd) with K / 128 even have
 * their whole 256-row tiles computed by a 256 x 256-tile kernel launched first on the
 * same stream; the definition above holds either way (the same promotion order, so
 * bit-identical outputs in every tested case).  Unset or any other value: one kernel.
 * Groups above the small-tile size are cut into 192-row tiles when K <= 8192 (into
 * 128-row tiles for larger K and with FP8GG_BIG_TILES; gemm_fp8 takes whichever of the two
 * gives its M the shorter schedule); FP8GG_TILE_ROWS=128 or 192 in the environment (read
 * at each call) forces one where both are possible.  Every choice computes each output
 * with the same block products and promotion order: bit-identical results. */
int grouped_gemm_fp8(const uint8_t *A, const float *sA, const int32_t *a_rows, int a_row_div,
                     const uint8_t *B, const float *sB, const int32_t *offsets, int G,
                     int R_cap, int N, int K, int epilogue, moe_dtype out_dt, void *C,
                     float *sC, void *stream);

/* The same GEMM over the fixed-capacity ("masked") expert layout, the second of the
 * grouped layouts DeepGEMM offers beside the contiguous one (qidao123.com day 3; the
 * per-expert capacity of mooersco.com sec. 2.5): group g owns rows [g*cap, g*cap +
 * counts[g]) of A [G*cap, K] (counts on the device, clamped to [0, cap]); sA
 * [G*cap, K/128]; C and sC have G*cap rows, rows past counts[g] in each block are
 * unspecified.  No row gather.  B, sB, epilogue, out_dt and sizes as grouped_gemm_fp8;
 * G * cap * K <= 2^32 - 256. */
int grouped_gemm_fp8_masked(const uint8_t *A, const float *sA, const uint8_t *B,
                            const float *sB, const int32_t *counts, int G, int cap, int N,
                            int K, int epilogue, moe_dtype out_dt, void *C, float *sC,
                            void *stream);

/* Dense FP8 GEMM with the same block scaling (the dense layout, qidao123.com day 3):
 * C [M, N] bf16 = A [M, K] e4m3 (sA [M, K/128]) times B [N, K] e4m3 (sB [N/128, K/128],
 * codes fragment-major as moe_pack_weight_fp8 with G = 1) transposed, promoted per
 * 128-deep K block.  N and K multiples of 128, K <= 16384, M * K <= 2^32 - 256,
 * M >= 0 (M = 0: nothing is launched, A, sA and C may be null).  C must not overlap sB (checked) nor A, sA, B. */
int gemm_fp8(const uint8_t *A, const float *sA, const uint8_t *B, const float *sB, int M,
             int N, int K, uint16_t *C, void *stream);

/* Rearranges int4 weights (codes q [G, N, K/2] and scales s7 [G, N, K/128] as
 * moe_quant_weight_int4 writes them) into the fragment-major order grouped_gemm_w4a8
 * loads: qf [G][N/16][K/128][64][16 B], lane l of 16-row block nb and 128-deep block kb
 * holding the 32 codes of row 16 nb + (l mod 16), k = 128 kb + 32 (l div 16) .. +32
 * (bytes 64 kb + 16 (l div 16) .. +16 of that row); s7f [G][N/16][K/128][16], the
 * scales of a block's 16 rows together.  A pure permutation, done once per weight.
 * Outputs must not overlap inputs; N and K multiples of 128.  (Layout of this library,
 * not of the pages.) */
int moe_pack_weight_int4(const uint8_t *q, const float *s7, int G, int N, int K, uint8_t *qf,
                         float *s7f, void *stream);

/* Grouped GEMM with 4-bit weights on the FP8 matrix core (W4A8).  The weights are the
 * block-wise 4-bit codes of the DeepSeek-V4 lecture (tqpw.cn sec. 3.1: q = round(w /
 * max|w| * 7) in [-7, 7] per output channel and 128-wide K block, s7 = max|w| / 7), kept
 * 4-bit in memory and fed to the e4m3 matrix instruction, on which the integers -7..7
 * are exact; the activations are 1x128 e4m3 as in grouped_gemm_fp8.  Each 128-deep block
 * is promoted as acc += sA[a, kb] * s7[g, n, kb] * partial (two-level accumulation,
 * qidao123.com day 3).  B and s7 as packed by moe_pack_weight_int4 ([G, Nb, K] logical,
 * Nb = N or 2N for SwiGLU); every other argument, output and limit as grouped_gemm_fp8.
 * Kernel choice as grouped_gemm_fp8, except that groups of at most ~170 rows (R_cap / G)
 * are cut into 160-row tiles (FP8GG_TILE_ROWS=160 forces them): bit-identical results. */
int grouped_gemm_w4a8(const uint8_t *A, const float *sA, const int32_t *a_rows, int a_row_div,
                      const uint8_t *B, const float *s7, const int32_t *offsets, int G,
                      int R_cap, int N, int K, int epilogue, moe_dtype out_dt, void *C,
                      float *sC, void *stream);

/* Grouped GEMM with int4 weights and bf16 activations (block-wise 4-bit expert weights
 * with max-abs scales, DeepSeek-V4 lecture, tqpw.cn, sec. 3.1; groups as in the
 * MegaMoE walkthrough, discosf.com, sec. 3.2): B codes [G, Nb, K/2] and
 * s7 [G, Nb, K/128] are dequantised in-kernel to bf16(fl32(q * s7)) and multiplied with
 * A [*, K] bf16 in fp32.  Row gather and epilogues as grouped_gemm_fp8; output C
 * [R_cap, N] bf16.  N and K multiples of 128. */
int grouped_gemm_w4a16(const uint16_t *A, const int32_t *a_rows, int a_row_div,
                       const uint8_t *B, const float *s7, const int32_t *offsets, int G,
                       int R_cap, int N, int K, int epilogue, uint16_t *C, void *stream);

/* Grouped fp32 GEMM (no quantisation; groups differ in M and share N and K, MegaMoE
 * walkthrough, discosf.com, sec. 3.2, written as a loop of per-expert GEMMs in the
 * Dense-to-TP-MoE article, cf-1.com, sec. 4.2): A [*, K] fp32, B [G, Nb, K] fp32, C [R_cap, N]
 * fp32.  Row gather and epilogues as grouped_gemm_fp8.  N multiple of 16, K >= 1. */
int grouped_gemm_f32(const float *A, const int32_t *a_rows, int a_row_div, const float *B,
                     const int32_t *offsets, int G, int R_cap, int N, int K, int epilogue,
                     float *C, void *stream);

/* Weighted combine (y = sum over the top-k of G(x)_i E_i(x), discosf.com sec. 2.1):
 * y[t] = sum_j topk_w[t,j] * o[row_of_slot[t*k+j]] in fp32, j = 0..k-1 in order,
 * slots with row -1 skipped; o [*, d] and y [T, d] of dtype MOE_BF16 or MOE_F32.
 * d a multiple of 8.  A deterministic gather: no atomics. */
int moe_combine(const void *o, moe_dtype o_dt, const int32_t *row_of_slot,
                const float *topk_w, int T, int k, int d, void *y, moe_dtype y_dt,
                void *stream);

typedef struct {
  int T, d, E, k, I;       /* tokens, hidden, experts, top-k, expert intermediate size */
  int mode;                /* MOE_MODE_*                                            */
  int route;               /* MOE_ROUTE_SCORE or MOE_ROUTE_HASH (k must be 1)       */
  unsigned route_flags;    /* MOE_ROUTE_RENORM                                      */
  double capacity_factor;  /* <= 0: dropless; > 0: capacity C = moe_capacity(T, k,  */
                           /* E, capacity_factor), which must be >= 1 when T > 0    */
  int m_align;             /* row padding quantum of each expert (1..1024)          */
  int layout;              /* MOE_LAYOUT_CONTIGUOUS, or MOE_LAYOUT_MASKED (FP8 mode  */
                           /* with capacity_factor > 0: buffers [E, C, *], C =      */
                           /* moe_capacity(T, k, E, capacity_factor))               */
} moe_layer_desc;

typedef struct {
  const void *w_router;    /* [E, d]: bf16 (FP8/W4A16 modes) or fp32 (FP32 mode)    */
  const float *bias;       /* [E] fp32 (score routing)                              */
  const void *w13;         /* [E, 2I, d]: rows [0,I) gate, [I,2I) up.  fp32 | e4m3  */
                           /*   fragment-major (moe_pack_weight_fp8) | int4 packed    */
                           /*   [E, 2I, d/2] (W4A8: moe_pack_weight_int4 order)       */
  const float *s13;        /* FP8: [E, 2I/128, d/128]; W4A16: [E, 2I, d/128];       */
                           /*   W4A8: packed by moe_pack_weight_int4                */
  const void *w2;          /* [E, d, I] (e4m3: fragment-major; int4: [E, d, I/2])   */
  const float *s2;         /* FP8: [E, d/128, I/128]; W4A16: [E, d, I/128]; W4A8    */
} moe_layer_weights;

/* Bytes of device workspace moe_layer_fwd needs for `desc` (0 on a bad descriptor;
 * MOE_MODE_FP8 also needs T * d and moe_rows_bound(T, k, E, m_align) * I <= 2^32 - 256,
 * the GEMMs' 32-bit operand offsets). */
size_t moe_layer_workspace_size(const moe_layer_desc *desc);

/* The whole layer forward on one stream, no host synchronisation:
 * route -> dispatch -> (FP8: per-token 1x128 quant) -> grouped GEMM1 with SwiGLU
 * (FP8: requantised 1x128) -> grouped GEMM2 -> combine: y = sum over the top-k experts
 * of G(x)_i E_i(x) with E_i a SwiGLU FFN (MegaMoE walkthrough, discosf.com, sec.
 * 2.1-2.2 and 3.2-3.3; hash routing and 4-bit weights, DeepSeek-V4 lecture, tqpw.cn,
 * sec. 2.2 and 3.1; capacity drop, DeepSeek MoE architecture, mooersco.com, sec. 2.5).
 *   x [T, d]: fp32 (FP32 mode) or bf16; token_ids [T] int64 for hash routing (x, y and
 *   token_ids may be NULL when T = 0);
 *   y [T, d] output: fp32 (FP32 mode) or bf16;
 *   ws / ws_bytes: caller-owned device workspace (>= moe_layer_workspace_size);
 *   counts_out [E] int32 (may be NULL): routed slots per expert (all 0 when T = 0).
 * Contiguous layout: GEMM1 reads activation rows through the dispatch map, so no
 * gathered copy of the activations is made.  Masked layout: moe_dispatch_masked, the
 * token codes gathered into the [E, C, d] buffer (1x128 quantisation, empty rows zero),
 * the masked GEMM1 and GEMM2 over counts clamped to C, then the combine. */
int moe_layer_fwd(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                  const int64_t *token_ids, void *y, void *ws, size_t ws_bytes,
                  int32_t *counts_out, void *stream);

/* Bytes of device workspace moe_layer_fwd_chunked needs for `desc` and `chunk_tokens`
 * (0 on a bad descriptor, a capacity, or the masked layout). */
size_t moe_layer_chunked_workspace_size(const moe_layer_desc *desc, int chunk_tokens);

/* The layer forward as a two-stream pipeline over token chunks (the chunked overlap of
 * the MegaMoE walkthrough, discosf.com, sec. 2.3 and 4.3: 128- or 256-token chunks; the
 * streams-and-events pattern of the Dense-to-TP-MoE article, cf-1.com, sec. 4.3): the
 * batch is cut into chunks of `chunk_tokens` tokens (the last one ragged); chunk i's
 * route, dispatch and token quantisation run on `stream_aux` while chunk i-1's expert
 * GEMMs and combine run on `stream`, ordered by events, with two workspace regions
 * alternating between chunks.  Each chunk is an independent layer pass, so y is the
 * layer's output (routing per token does not depend on the chunking; the router's
 * split-K order, and with it the last bits of the gate weights, may).  Every chunk
 * streams the touched experts' weights again: on one GPU, where there is no all-to-all to
 * hide, this costs about one weight stream per chunk.  Dropless contiguous layout only
 * (capacity_factor <= 0).  stream_aux must differ from stream; it starts after the work
 * enqueued on `stream` before the call, and `stream` ends after all of the call's work.
 * counts are not reported.  Arguments otherwise as moe_layer_fwd. */
int moe_layer_fwd_chunked(const moe_layer_desc *desc, const moe_layer_weights *w, const void *x,
                          const int64_t *token_ids, void *y, void *ws, size_t ws_bytes,
                          int chunk_tokens, void *stream, void *stream_aux);

/* ---- measurement probes (not part of the layer's computation) ----
 * References for the rooflines the layer's kernels are measured against: the rates the
 * FP8 matrix core and the HBM read path reach on this device, beside the datasheet
 * peaks.  Both enqueue one kernel of n_blocks workgroups of 512 threads on `stream`;
 * the caller times it (HIP events on `stream`). */

/* FP8 matrix-core issue rate.  Every wave runs `iters` rounds of four independent
 * 16x16x128 e4m3 MFMAs (the FP8 GEMMs' instruction) on operands whose bytes all equal
 * `code` (an e4m3 code, not a NaN), so the call performs n_blocks * 8 * iters * 4 *
 * 65536 FLOP.  out: device fp32 [n_blocks * 512], fully written; lane i's value is
 * 2048 * iters * v^2 for the code's value v (exact while 128 * iters * v^2 < 2^24).
 * n_blocks in [1, 65536] (one per CU runs two waves per SIMD, as the GEMMs do),
 * iters >= 1. */
int moe_probe_mfma_fp8(int n_blocks, int iters, uint8_t code, float *out, void *stream);

/* HBM read rate.  Reads the `bytes` bytes at `buf` (device, 16-byte aligned, bytes a
 * positive multiple of 16) once with 16-byte non-temporal loads, grid-strided over
 * n_blocks workgroups (n_blocks in [1, 65536]); out: device uint32 [n_blocks], fully
 * written, the XOR of the 32-bit words that workgroup read (so the XOR over out is the
 * XOR of the whole buffer). */
int moe_probe_hbm_read(const void *buf, size_t bytes, int n_blocks, uint32_t *out,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8GG_MOE_H */
