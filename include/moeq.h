/*
 * moeq.h - C ABI of the quantized mixture-of-experts grouped GEMM library
 *          for AMD Instinct MI355X (gfx950).
 *
 * The routed MoE hot path in five calls:
 *   moe_route_prep          group (token, slot) pairs by expert
 *   grouped_gemm_qint4      W4A4 INT4 GEMM, per-token x per-channel scales
 *   grouped_gemm_qfp8_block FP8 e4m3 GEMM, 1x128 A / 128x128 B block scales
 *   grouped_gemm_qnvfp4     NVFP4 (E2M1 + UE4M3 per-16 + global) x bf16 GEMM
 *   moe_scatter_combine     top-k weighted sum back to token rows
 *   (or: grouped_gemm_qnvfp4 with pair_weights + moe_sum_pairs, the top-k
 *   weight applied in FC2's epilogue)
 * with helpers around it:
 *   moe_quantize_int4       per-row INT4 activation quantization
 *   moe_nvfp4_repack        one-shot NVFP4 weight layout conversion
 *   moe_cast_bf16_to_f16    activations for the binary16 NVFP4 form
 *   moe_route_prep_noalloc  route prep for callers that cannot allocate
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer (memory the caller allocated
 *     on the current HIP device) unless marked "host".  The caller owns all
 *     memory, scratch included (route prep's workspace, the NVFP4 work
 *     queue); the library allocates nothing and never synchronizes the host
 *     with the device.  Its state is moe_route_prep_noalloc's fixed
 *     per-device scratch and a per-device cache of the compute-unit count
 *     (read once from the HIP runtime; safe to fill from several threads).
 *   - Every call only validates its arguments on the host and enqueues
 *     kernels on `stream` (a hipStream_t; NULL = the null stream).  Results
 *     are visible to later work on that stream.
 *   - Argument errors are detected before anything is enqueued and returned
 *     as a status; moeq_last_error() then gives a text for the calling
 *     thread.  A failed launch returns MOEQ_EHIP.  Nothing throws.
 *   - Shorthands: T tokens, topk = k slots per token, E experts,
 *     P = T*topk pairs, pair id p = t*topk + j for topk_ids[t][j].
 *   - 4-bit codes (INT4 and E2M1) are packed two per byte, element 2b in the
 *     low nibble of byte b.  Matrices are row-major; a weight matrix W[e] is
 *     stored [N][K] with K contiguous (y = x . W^T).
 *   - Grouped GEMM rows: sorted position s in [0, expert_offsets[E]) belongs
 *     to expert e with expert_offsets[e] <= s < expert_offsets[e+1]; its
 *     output row is out[s][:].  Rows past expert_offsets[E] are not written.
 *     The activation row used for s is chosen by moeq_arow:
 *       MOEQ_AROW_TOKEN : row sorted_pair_ids[s] / topk  (token-major input
 *                         [T][K], each token feeding its k experts)
 *       MOEQ_AROW_SORTED: row s  (input already in sorted order, e.g. the
 *                         output of a previous grouped GEMM)
 *     With sorted_pair_ids == NULL the rows are the identity (SORTED).
 *
 * Sources (web pages on quantized MoE grouped GEMMs; cited by title):
 *   [W4A4]   CUTLASS discussion #2855, "How to implement dequantization of
 *            row and column broadcast in Epilogue of GroupGemm"
 *   [FP8BLK] CUTLASS issue #2087, "how to use groupwise scaling along M for
 *            FP8 gemm to implement per-token-per-128-channel and blockwise"
 *   [TLK]    nvfp4-megamoe-kernel, tilelang_kernels.py (grouped_gemm_fp4)
 *   [MMRM]   megamoe_rm.cu (route_prep, fc1_rm, fc2_rm, combine)
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOEQ_OK = 0,
  MOEQ_EINVAL = 1,       /* null pointer, negative or inconsistent size */
  MOEQ_EALIGN = 2,       /* pointer or dimension not aligned as required */
  MOEQ_EUNSUPPORTED = 3, /* dtype / act / mode combination not provided */
  MOEQ_EHIP = 4          /* a HIP launch failed */
} moeq_status;

typedef enum { MOEQ_F16 = 1, MOEQ_BF16 = 2, MOEQ_F32 = 3, MOEQ_I32 = 4 } moeq_dtype;

/* MOEQ_ACT_SILU_MUL: the GEMM's N = 2I columns are [gate | up]
 * (columns [0, I) gate, [I, 2I) up); the call writes I columns
 * h = silu(gate) * up, silu(g) = g / (1 + exp(-g)).
 * MOEQ_ACT_SILU_MUL_LIMIT (grouped_gemm_qnvfp4 only): the clamped form of
 * [MMRM] fc1_rm's epilogue, applied to the scaled outputs before the
 * product: gate = min(gate, limit), up = min(max(up, -limit), limit). */
typedef enum { MOEQ_ACT_NONE = 0, MOEQ_ACT_SILU_MUL = 1, MOEQ_ACT_SILU_MUL_LIMIT = 2 } moeq_act;

typedef enum { MOEQ_AROW_TOKEN = 0, MOEQ_AROW_SORTED = 1 } moeq_arow;

/* Layout of NVFP4 block scales (C = K/16 per row).
 * MOEQ_SF_ROWS   [E][N][C] row-major, the layout of [TLK].
 * MOEQ_SF_KQUADS [E][C/4][N][4]: for each group of 4 block columns (64
 *                values of K), the 4 scale bytes of every row, rows
 *                consecutive.  A K step of 64 finds the scales of
 *                consecutive weight rows in one contiguous run, which the
 *                tiled schedule fetches as whole cache lines; byte (n, c) is
 *                at ((c/4)*N + n)*4 + c%4 within an expert.
 * moe_nvfp4_repack produces either one. */
typedef enum { MOEQ_SF_ROWS = 0, MOEQ_SF_KQUADS = 1 } moeq_sf_layout;

/* Layout of NVFP4 E2M1 codes.
 * MOEQ_W_ROWS  [E][N][K/2] row-major.
 * MOEQ_W_TILED each expert's [N][K/2] bytes in blocks of 16 rows x 32
 *              bytes (64 values of K), 512 bytes each, a 16-row group's
 *              blocks consecutive along K: byte (n, b) of an expert at
 *              ((n/16)*(K/64) + b/32)*512 + (n%16)*32 + b%32.  The tiled
 *              schedule then reads whole lines of codes, and a row group's
 *              codes stay one contiguous run for the streaming schedule.
 * moe_nvfp4_repack produces either one. */
typedef enum { MOEQ_W_ROWS = 0, MOEQ_W_TILED = 1 } moeq_w_layout;

/* Schedule hint for the grouped GEMMs.  Both schedules compute the same
 * result for every input; AUTO picks by the average rows per expert
 * (P / E): the weight-streaming DECODE schedule for few rows per expert,
 * the MFMA-tiled PREFILL schedule otherwise. */
typedef enum { MOEQ_SCHED_AUTO = 0, MOEQ_SCHED_DECODE = 1, MOEQ_SCHED_PREFILL = 2 } moeq_sched;

/* Text describing the last non-OK status returned on the calling thread
 * (host, thread-local, owned by the library; valid until the next call). */
const char* moeq_last_error(void);

/* int32 counters of grouped_gemm_qnvfp4's optional work queue. */
#define MOEQ_WORK_QUEUE_INTS 16

/* Library ABI version (host). */
int32_t moeq_abi_version(void);

/* ------------------------------------------------------------------------
 * moe_route_prep - group the P = T*topk (token, slot) pairs by expert.
 * [MMRM] route_prep (pair id token*topk + k; a pair's place is its rank
 * among earlier pairs of the same expert, so the table is unique; id -1
 * means no expert); [W4A4] the [E+1] per-expert row-offset table.
 *
 *   topk_ids        int32 [T][topk]   expert id per slot; -1 = none
 *   expert_offsets  int32 [E+1] out   exclusive prefix of per-expert counts
 *   sorted_pair_ids int32 [P]   out   valid pairs ordered by (expert, pair
 *                                     id); positions >= expert_offsets[E]
 *                                     hold -1
 *   pair_to_sorted  int32 [P]   out   inverse: sorted position of pair p,
 *                                     -1 if p was skipped
 *   n_invalid       int32 [1]   out   number of ids outside [0, E) other
 *                                     than -1 (those pairs are skipped too)
 *   workspace       device scratch of moe_route_prep_workspace_bytes() bytes
 *                   (may be NULL when that is 0); contents on entry ignored
 * Requires T >= 0, 1 <= topk <= 64, 1 <= E <= 1024, T*topk < 2^31.
 * T == 0 writes expert_offsets = 0 and n_invalid = 0.
 * moe_route_prep_workspace_bytes returns 0 for arguments outside these
 * ranges (the call itself then gives MOEQ_EINVAL).
 * ---------------------------------------------------------------------- */
size_t moe_route_prep_workspace_bytes(int64_t T, int32_t topk, int32_t E); /* host */

moeq_status moe_route_prep(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                           int32_t* expert_offsets, int32_t* sorted_pair_ids,
                           int32_t* pair_to_sorted, int32_t* n_invalid, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_route_prep_noalloc - moe_route_prep for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same tables, with the per-chunk
 * counts kept in a fixed device array of the library instead of a
 * caller's workspace.
 *
 * Arguments, outputs and checks as moe_route_prep, without the workspace.
 * The array holds MOEQ_ROUTE_NOALLOC_SCRATCH_BYTES per GPU, so the call
 * serves T*topk pairs while moe_route_prep_workspace_bytes(T, topk, E) is
 * at most that (e.g. E = 256: about 10^6 pairs); larger sizes give
 * MOEQ_EINVAL.  Each GPU holds its own array from the first call made with
 * that device current (which looks up its address) until the process
 * ends.  Every call on one GPU uses the same array: calls that overlap in
 * time on one GPU (different streams, or different host threads) race and
 * give undefined tables; calls ordered on one stream do not.  The array
 * needs no clearing (each call writes every count it later reads).  The
 * call allocates nothing and never synchronizes.
 * ---------------------------------------------------------------------- */
#define MOEQ_ROUTE_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)

moeq_status moe_route_prep_noalloc(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                                   int32_t* expert_offsets, int32_t* sorted_pair_ids,
                                   int32_t* pair_to_sorted, int32_t* n_invalid, void* stream);

/* ------------------------------------------------------------------------
 * grouped_gemm_qint4 - W4A4 INT4 grouped GEMM with the dequantization fused
 * into the epilogue.  [W4A4] problem statement: activations quantized per
 * token, weights per output channel, int32 accumulation,
 * y = scale_act * scale_weight * accumulator.
 *
 *   a          uint8 [rows_a][K/2]   int4 activations (two's complement)
 *   a_scale    f32   [rows_a]        per-row activation scale
 *   w          uint8 [E][N][K/2]     int4 weights
 *   w_scale    f32   [E][N]          per-output-channel weight scale
 *   expert_offsets, sorted_pair_ids  from moe_route_prep (see top)
 *   P          rows of `out` (>= expert_offsets[E]); topk as routed
 *   out        [P][N] (act NONE) or [P][N/2] (SILU_MUL) of out_dtype:
 *                F16 | BF16 | F32: a_scale[r] * w_scale[e][n] * acc
 *                I32: the raw accumulator acc (act NONE only), bit-exact
 * Computed exactly in integers (int8 MFMA on nibbles scaled by 16), then
 * scaled in fp32 and rounded to nearest even.
 * Requires K % 128 == 0 and N % 32 == 0 (else MOEQ_EALIGN; [W4A4]'s
 * launcher checks K and N against 32; SILU_MUL then writes I = N/2 columns,
 * a multiple of 16), K < 131072 so that the int32 accumulator cannot wrap
 * (else MOEQ_EINVAL), all pointers 16-byte aligned, 1 <= E <= 1024,
 * 1 <= topk <= 64.
 * Two schedules give identical outputs: 256x256 MFMA tiles (PREFILL), and
 * waves streaming 32 weight rows x at most 8 routed rows of one expert
 * (DECODE), which needs K % 256 == 0 (else MOEQ_EALIGN).  AUTO streams when
 * K % 256 == 0 and either P < 16 * E or the tiles would be fewer than half
 * the compute units.
 * ---------------------------------------------------------------------- */
moeq_status grouped_gemm_qint4(const uint8_t* a, const float* a_scale, int64_t rows_a,
                               moeq_arow a_row, const uint8_t* w, const float* w_scale,
                               const int32_t* expert_offsets, const int32_t* sorted_pair_ids,
                               int64_t P, int32_t topk, int32_t E, int64_t N, int64_t K,
                               moeq_act act, moeq_dtype out_dtype, void* out, moeq_sched sched,
                               void* stream);

/* ------------------------------------------------------------------------
 * grouped_gemm_qfp8_block - FP8 e4m3 block-scaled grouped GEMM.  [FP8BLK]:
 * A scaled per token per 128 columns of K, B per 128x128 block; scales
 * applied per 128-wide K group inside the main loop (fp32 accumulation).
 *
 *   a        uint8 [rows_a][K]        OCP e4m3fn activations
 *   a_scale  f32   [K/128][rows_a]    per (K group, row); rows contiguous,
 *                                     the M-contiguous layout [FP8BLK]
 *                                     recommends so scale loads coalesce
 *   w        uint8 [E][N][K]          OCP e4m3fn weights
 *   w_scale  f32   [E][N/128][K/128]  per 128x128 weight block
 *   out      [P][N] out_dtype (BF16 | F16 | F32)
 *   y[s][n] = sum_g a_scale[g][r] * w_scale[e][n/128][g]
 *                   * sum_{k in group g} a[r][k] * w[e][n][k]
 * Requires K % 128 == 0 and N % 128 == 0 (else MOEQ_EALIGN), 16-byte
 * aligned pointers, 1 <= E <= 1024, 1 <= topk <= 64.  sched AUTO takes the
 * weight-streaming schedule (waves streaming 16 weight rows x at most 4
 * routed rows) when P < 16 * E, the 128x128 MFMA tiles otherwise; both
 * compute the same sums, grouped per 128-wide K block as above.
 * ---------------------------------------------------------------------- */
moeq_status grouped_gemm_qfp8_block(const uint8_t* a, const float* a_scale, int64_t rows_a,
                                    moeq_arow a_row, const uint8_t* w, const float* w_scale,
                                    const int32_t* expert_offsets,
                                    const int32_t* sorted_pair_ids, int64_t P, int32_t topk,
                                    int32_t E, int64_t N, int64_t K, moeq_dtype out_dtype,
                                    void* out, moeq_sched sched, void* stream);

/* ------------------------------------------------------------------------
 * grouped_gemm_qnvfp4 - NVFP4 W4A16 grouped GEMM.  [TLK] grouped_gemm_fp4
 * (E2M1 weights with UE4M3 scales per 16 along K, bf16 activations) with
 * the per-expert global scale of [MMRM] (alpha = weight_scale_2 /
 * input_scale).  Weights are dequantized exactly (every E2M1 x UE4M3
 * product is both a bf16 and a binary16 value) in registers, never as a
 * separate pass.
 *
 *   x         [rows_a][K] activations of x_dtype: BF16, or F16 ([MMRM]'s
 *             fp16 activations; the weights are then dequantized and
 *             multiplied in fp16, at half the dequantization work; see
 *             moe_cast_bf16_to_f16)
 *   w         uint8 E2M1 codes in w_layout: [E][N][K/2] (ROWS) or tiled
 *             (TILED, faster for the tiled schedule), E*N*K/2 bytes
 *   w_sf      uint8 UE4M3 block scales (sign bit clear; 0x7F is not a
 *             valid scale) in sf_layout: [E][N][K/16] (ROWS) or
 *             [E][K/64][N][4] (KQUADS, faster for the tiled schedule).
 *             [TLK]'s uint32 [E][N][K/64] packing (block 4g+j in bits
 *             8j..8j+7 of word g) is the ROWS bytes and may be passed as is
 *   w_gscale  f32   [E]               per-expert global scale
 *   act       NONE, SILU_MUL, or SILU_MUL_LIMIT with act_limit (host f32,
 *             > 0, +inf allowed; ignored for the other acts; a NaN, zero
 *             or negative limit gives MOEQ_EINVAL)
 *   pair_weights  NULL, or f32 [P] indexed by pair id (topk_weights
 *             flattened): [MMRM] fc2_rm's epilogue.  Sorted row s is then
 *             multiplied by pair_weights[p], p = sorted_pair_ids[s], and
 *             written to out row p (pair order) instead of row s; rows of
 *             pairs without an expert are not written.  Needs act NONE
 *             (else MOEQ_EUNSUPPORTED) and sorted_pair_ids (else
 *             MOEQ_EINVAL); every pair id must be < P, as moe_route_prep's
 *             are.  moe_sum_pairs then sums each token's rows.
 *   out       [P][N] (NONE) or [P][N/2] (SILU_MUL*), BF16 | F16 | F32
 *   work_queue  NULL, or MOEQ_WORK_QUEUE_INTS int32 of device memory, 4-byte
 *             aligned (else MOEQ_EALIGN), that are zero when the call starts
 *             running (zero them once: every call leaves them zero).  The
 *             tiled schedule then hands its tiles out through atomic
 *             counters in them (one per XCD), so a workgroup takes the next
 *             tile when it finishes one, which balances tiles of unequal
 *             cost (the partial last m-tiles of skewed routing); without it
 *             each workgroup takes every gridDim-th tile.  The outputs are
 *             the same either way.  Calls that may overlap in time on one
 *             GPU need separate queues.  The streaming schedule ignores it.
 *   y[s][n] = w_gscale[e] * sum_k x[r][k] * e2m1(w[e][n][k])
 *                                  * ue4m3(w_sf[e][n][k/16])
 * Requires K % 128 == 0 and N % 32 == 0 (else MOEQ_EALIGN; SILU_MUL then
 * writes I = N/2 columns, a multiple of 16), 16-byte aligned pointers,
 * 1 <= E <= 1024, 1 <= topk <= 64.  sched AUTO takes the weight-streaming
 * schedule when P < 16 * E or N % 256 != 0; PREFILL with N % 256 != 0
 * falls back to it as well.
 * ---------------------------------------------------------------------- */
moeq_status grouped_gemm_qnvfp4(const void* x, moeq_dtype x_dtype, int64_t rows_a, moeq_arow a_row,
                                const uint8_t* w, moeq_w_layout w_layout, const uint8_t* w_sf,
                                moeq_sf_layout sf_layout, const float* w_gscale,
                                const int32_t* expert_offsets, const int32_t* sorted_pair_ids,
                                int64_t P, int32_t topk, int32_t E, int64_t N, int64_t K,
                                moeq_act act, float act_limit, const float* pair_weights,
                                moeq_dtype out_dtype, void* out, int32_t* work_queue, moeq_sched sched,
                                void* stream);

/* ------------------------------------------------------------------------
 * moe_cast_bf16_to_f16 - bf16 -> IEEE binary16 conversion of activations,
 * for the F16 form of grouped_gemm_qnvfp4 ([MMRM] route_prep converts its
 * bf16 input to fp16 the same way).  Each value is rounded once to the
 * nearest binary16 (ties to even, overflow to +-inf), so every bf16 value
 * of magnitude in [2^-14, 65504] converts exactly.
 *
 *   x  uint16 [n] bf16 bits;  y  uint16 [n] binary16 bits (out)
 * Requires n % 8 == 0 (else MOEQ_EALIGN), 16-byte aligned x and y, and y
 * either equal to x (in place) or disjoint from it (else MOEQ_EINVAL).
 * ---------------------------------------------------------------------- */
moeq_status moe_cast_bf16_to_f16(const uint16_t* x, int64_t n, uint16_t* y, void* stream);

/* ------------------------------------------------------------------------
 * moe_quantize_int4 - per-row symmetric INT4 quantization of activations.
 * [W4A4] quantizes the fp16 activations per token to int4 (the token scale
 * is then applied with the channel scale in the GEMM epilogue); the page
 * gives no rounding rule, the one used is:
 *   amax = max_k |x[r][k]|,  scale[r] = amax / 7,
 *   code = clamp(rne(x[r][k] * (7 / amax)), -8, 7)
 * with each division and the product one fp32 operation; a row with
 * amax < 2^-120 (an all-zero row included) gives zeros and scale 1.
 *
 *   x      [rows][K] x_dtype (F16 | BF16 | F32), rows contiguous
 *   q      uint8 [rows][K/2]  two's-complement codes, element 2b in the
 *          low nibble of byte b (grouped_gemm_qint4's activation layout)
 *   scale  f32 [rows]
 * Requires K % 16 == 0 (else MOEQ_EALIGN), x and q 16-byte aligned, scale
 * 4-byte aligned.  NaN or infinite inputs give unspecified codes.
 * ---------------------------------------------------------------------- */
moeq_status moe_quantize_int4(const void* x, moeq_dtype x_dtype, int64_t rows, int64_t K, uint8_t* q,
                              float* scale, void* stream);

/* ------------------------------------------------------------------------
 * moe_scatter_combine - weighted sum of each token's expert rows.
 * [MMRM] combine (a token's pairs that have an expert, summed in slot
 * order in fp32, one rounding); [TLK] zero output plus weighted
 * scatter-add.
 *
 *   y             [P][N] y_dtype (F16 | BF16 | F32), rows in sorted order
 *   pair_to_sorted int32 [T*topk] from moe_route_prep
 *   topk_weights  f32 [T][topk]
 *   out           [T][N] out_dtype (F16 | BF16 | F32)
 *   out[t][:] = sum_{j < topk, pair_to_sorted[t*topk+j] >= 0}
 *                 topk_weights[t][j] * y[pair_to_sorted[t*topk+j]][:]
 * accumulated in fp32 in slot order and rounded once (nearest even);
 * a token with no routed pair gets a zero row.
 * Requires N % 8 == 0, 16-byte aligned pointers.
 * ---------------------------------------------------------------------- */
moeq_status moe_scatter_combine(const void* y, moeq_dtype y_dtype, const int32_t* pair_to_sorted,
                                const float* topk_weights, int64_t T, int32_t topk, int64_t N,
                                moeq_dtype out_dtype, void* out, void* stream);

/* ------------------------------------------------------------------------
 * moe_sum_pairs - per-token sum of pre-weighted rows in pair order.
 * [MMRM] combine: the rows fc2_rm's epilogue wrote (grouped_gemm_qnvfp4
 * with pair_weights) summed over a token's pairs that have an expert, in
 * slot order, in fp32, rounded once.
 *
 *   y_pairs        [T*topk][N] y_dtype (F16 | BF16 | F32), row t*topk + j
 *   pair_to_sorted int32 [T*topk] from moe_route_prep (< 0: no expert, the
 *                  row is skipped and need not hold a value)
 *   out            [T][N] out_dtype (F16 | BF16 | F32)
 *   out[t][:] = sum_{j < topk, pair_to_sorted[t*topk+j] >= 0}
 *                 y_pairs[t*topk+j][:]
 * A token with no routed pair gets a zero row.  Requires N % 8 == 0,
 * 16-byte aligned y_pairs and out, 1 <= topk <= 64.
 * ---------------------------------------------------------------------- */
moeq_status moe_sum_pairs(const void* y_pairs, moeq_dtype y_dtype, const int32_t* pair_to_sorted, int64_t T,
                          int32_t topk, int64_t N, moeq_dtype out_dtype, void* out, void* stream);

/* ------------------------------------------------------------------------
 * moe_nvfp4_repack - convert NVFP4 expert weights from the layout [MMRM]
 * reads in place (its header comment and scale_off) to the layout of
 * grouped_gemm_qnvfp4.  One-shot, at weight-load time.
 *
 *   w_in    uint8 [E][N][K/2]   E2M1 codes, rows as stored for [MMRM]
 *   sf_in   uint8 [E][N*K/16]   UE4M3 scales of each expert's [N][K/16]
 *                               scale matrix in 128x4 tiles: the byte of
 *                               row r, block column c sits at
 *                                 ((r/128)*(K/64) + c/4) * 512
 *                                 + (r%32)*16 + ((r/32)%4)*4 + c%4
 *   swap_halves  0: rows keep their order (a w2 / down projection);
 *                1: the matrix is a w13 with the up rows [0, N/2) first
 *                   and the gate rows [N/2, N) second; the output puts the
 *                   gate rows first, the order of MOEQ_ACT_SILU_MUL
 *   w_out_layout MOEQ_W_ROWS or MOEQ_W_TILED: the layout of w_out
 *   out_layout   MOEQ_SF_ROWS or MOEQ_SF_KQUADS: the layout of sf_out
 *   w_out   uint8 [E*N*K/2]     out: the codes in w_out_layout, row n =
 *                               input row n (swap 0) or (n + N/2) mod N
 *                               (swap 1)
 *   sf_out  uint8 [E][N*K/16]   out: the scales in out_layout, rows as
 *                               w_out
 * A pure byte permutation: the outputs are bit-exact copies of input bytes.
 * Requires 1 <= E <= 1024, N % 128 == 0 and K % 64 == 0 (else MOEQ_EALIGN),
 * N*K < 2^36, all four pointers non-NULL and 16-byte aligned, and the two
 * outputs disjoint from each other and from the inputs (no in-place repack:
 * MOEQ_EINVAL).  The per-expert global scale needs no repack.
 * ---------------------------------------------------------------------- */
moeq_status moe_nvfp4_repack(const uint8_t* w_in, const uint8_t* sf_in, int64_t E, int64_t N, int64_t K,
                             int32_t swap_halves, moeq_w_layout w_out_layout, moeq_sf_layout out_layout,
                             uint8_t* w_out, uint8_t* sf_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ_H */
