/*
 * fp8q.h -- C ABI of the FP8 (E4M3) fine-grained block-quantisation and block-scaled GEMM
 * library for AMD Instinct MI355X (gfx950). Library file: libfp8q.so.
 *
 * The operations follow these pages (cited by title and section):
 *   - pomoai.com hub page "DeepSeek-V3", section "FP8 mixed-precision training": float8
 *     e4m3; weights stored as 128x128 blocks, each with one float32 scale factor
 *     (weight_scale_inv); activations quantised at run time per token per 128 channels;
 *     and the linear() listing in that section: act_quant(x, block_size) -> (x_fp8,
 *     scale), fp8_gemm(x, scale, weight, weight.scale) -> y (not re-quantised; the bias
 *     is added by the caller), weight_dequant(weight, weight.scale) -> high-precision
 *     weight.
 *   - qdgithub.com book 25/317, section "FP8 quantisation: balancing storage and
 *     compute": row/column blocking, FP8 inside each block, dequantisation outside the
 *     matrix units.
 *   - 88811315.cn post 75335, Float8-training paragraph: E4M3 only, FP8 partial products
 *     promoted into an FP32 main accumulator.
 *
 * Numeric conventions (the pages leave these open):
 *   E4M3      OCP E4M3FN: bias 7, largest finite 448 (0x7E), S.1111.111 = NaN, no inf.
 *   scale     s = RN_fp32(amax / 448) per tile/block (IEEE division); amax = max |x|.
 *   code      q = E4M3 round-to-nearest-even with saturation of RN_fp32(x / s); for an
 *             all-zero tile s = 0 is stored and the codes are signed zeros.
 *   dequant   w = RN_bf16(RN_fp32(decode(q) * s)).
 *   GEMM      Y[m,n] = sum_kb P[m,n,kb] * (sa[m,kb] * sw[n/128,kb]), where P is the fp32
 *             partial of the 128-wide K slice kb, accumulated in fp32.
 *   NaN and infinite inputs are outside the contract.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to caller-owned memory, row-major and
 *     contiguous. bf16 is passed as its uint16_t bit pattern, E4M3 as uint8_t, scales as
 *     float. The library never allocates, frees or keeps these pointers.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns without waiting. Results are valid once the stream has reached that point.
 *   - Arguments are validated on the host before anything is enqueued; on any error the
 *     call returns a non-zero FP8Q_ERR_* code and enqueues nothing. A failed launch
 *     returns FP8Q_ERR_LAUNCH. Faults during execution surface at the caller's stream
 *     synchronisation. No C++ exception crosses this interface.
 *   - Sizes are int64_t. K must be a non-negative multiple of 128. A zero M or N (or, for
 *     the quantisers, K) is a valid empty call that enqueues nothing; null pointers are
 *     then allowed.
 *   - The calls are stateless and may be issued concurrently from several host threads.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define FP8Q_OK 0
#define FP8Q_ERR_NULL 1        /* a required pointer is NULL                                */
#define FP8Q_ERR_SHAPE 2       /* negative size, K not a multiple of 128, or size too large */
#define FP8Q_ERR_ALIGN 3       /* pointer alignment below what the entry point requires     */
#define FP8Q_ERR_DTYPE 4       /* unknown output dtype                                      */
#define FP8Q_ERR_UNSUPPORTED 5 /* no gfx950 device is current                               */
#define FP8Q_ERR_LAUNCH 6      /* the kernel launch failed                                  */
#define FP8Q_ERR_WORKSPACE 7   /* more scratch needed than fp8_block_gemm_noalloc holds     */

/* Output dtypes of fp8_block_gemm (low 8 bits of its y_dtype argument). */
#define FP8Q_OUT_F32 0
#define FP8Q_OUT_BF16 1

/* Contraction mode of fp8_block_gemm, OR-ed into y_dtype (at most one; 0 = default).
 * FP8Q_GEMM_FP8_PRODUCTS: each 128-wide slice partial comes from the FP8 matrix unit. That
 *   unit forms the sum of every group of 8 consecutive k after aligning the products to the
 *   group's largest one with 13 fraction bits (measured on gfx950), so a product more than
 *   about 2^7 below its group's largest loses low-order bits. Fastest.
 * FP8Q_GEMM_EXACT_SLICES: the E4M3 operands are converted exactly to f16 in registers and
 *   each slice partial comes from the f16 matrix unit, exact up to fp32 rounding of the four
 *   32-wide partial sums. About half the FP8 rate.
 * Default: exact slices for fp32 output, FP8 products for bf16 output (where bf16 rounding
 *   dominates). */
#define FP8Q_GEMM_FP8_PRODUCTS 0x100
#define FP8Q_GEMM_EXACT_SLICES 0x200

/* Layout flag of fp8_block_gemm / fp8_block_gemm_bias, OR-ed into y_dtype: the activation
 * scales sa are K-block-major, [K/128, M] with sa[kb * M + m] (the layout of
 * fp8_act_quant_kmajor), instead of row-major [M, K/128]. The values are the same; in this
 * layout the scales of one K slice for consecutive rows are contiguous, so the GEMM fetches
 * them as whole cache lines. Requires M * (K/128) < 2^29 (FP8Q_ERR_SHAPE otherwise).
 * fp8_grouped_gemm and fp8_rowwise_gemm take row-major scales only (FP8Q_ERR_DTYPE). */
#define FP8Q_SA_KMAJOR 0x1000

/* fp8_act_quant -- per-token, per-128-channel activation quantisation.
 * (pomoai.com "DeepSeek-V3", FP8 section: dynamic activation quantisation per token per
 * 128 channels; act_quant in the linear() listing.)
 *   x  [M, K] bf16 input.                       16-byte aligned.
 *   q  [M, K] E4M3 output.                      16-byte aligned.
 *   s  [M, K/128] fp32 output; s[m, kb] is the scale of x[m, 128*kb : 128*kb + 128].
 *                                               4-byte aligned.
 * Every code and scale is bit-identical to the definition above. */
int fp8_act_quant(const uint16_t *x, uint8_t *q, float *s, int64_t M, int64_t K, void *stream);

/* fp8_act_quant_kmajor -- fp8_act_quant (same passage, same codes and scale values) with the
 * scales written K-block-major:
 *   s  [K/128, M] fp32; s[kb * M + m] is the scale of x[m, 128*kb : 128*kb + 128].
 *                                               4-byte aligned.
 * The input of fp8_block_gemm with FP8Q_SA_KMAJOR. Requires M * (K/128) < 2^29
 * (FP8Q_ERR_SHAPE otherwise); other arguments and errors as fp8_act_quant. */
int fp8_act_quant_kmajor(const uint16_t *x, uint8_t *q, float *s, int64_t M, int64_t K, void *stream);

/* fp8_weight_quant -- 128x128 block quantisation of a weight matrix.
 * (pomoai.com "DeepSeek-V3", FP8 section: FP8 weights in 128x128 blocks, one float32
 * scale factor per block.)
 *   w  [N, K] bf16 input.                       16-byte aligned.
 *   q  [N, K] E4M3 output.                      16-byte aligned.
 *   s  [ceil(N/128), K/128] fp32 output; s[nb, kb] is the scale of the block rows
 *      [128*nb, min(128*nb + 128, N)), columns [128*kb, 128*kb + 128). The last block row
 *      may be ragged (N not a multiple of 128); its amax covers the valid rows only.
 *                                               4-byte aligned. */
int fp8_weight_quant(const uint16_t *w, uint8_t *q, float *s, int64_t N, int64_t K, void *stream);

/* fp8_weight_dequant -- E4M3 weight and its block scales back to bf16.
 * (pomoai.com "DeepSeek-V3", the bf16 branch of linear(): weight_dequant(weight,
 * weight.scale); qdgithub.com 25/317: dequantise outside the matrix units.)
 *   q  [N, K] E4M3 input.                       16-byte aligned.
 *   s  [ceil(N/128), K/128] fp32 input (layout of fp8_weight_quant). 4-byte aligned.
 *   w  [N, K] bf16 output, w = RN_bf16(RN_fp32(decode(q) * s)). 16-byte aligned. */
int fp8_weight_dequant(const uint8_t *q, const float *s, uint16_t *w, int64_t N, int64_t K,
                       void *stream);

/* fp8_block_gemm -- Y = A . W^T on block-quantised operands with per-slice promotion.
 * y_dtype = FP8Q_OUT_F32 or FP8Q_OUT_BF16, optionally OR-ed with one FP8Q_GEMM_* mode and
 * with FP8Q_SA_KMAJOR.
 * (pomoai.com "DeepSeek-V3", linear(): fp8_gemm(x, scale, weight, weight.scale);
 * qdgithub.com 25/317: FP8 products inside each block, dequantisation outside the matrix
 * units; 88811315.cn 75335: FP8 partials promoted into an FP32 accumulator.)
 *   aq [M, K] E4M3 activations, sa [M, K/128] fp32   (layout of fp8_act_quant), or
 *      with FP8Q_SA_KMAJOR sa [K/128, M]            (layout of fp8_act_quant_kmajor)
 *   wq [N, K] E4M3 weights,     sw [ceil(N/128), K/128] fp32 (layout of fp8_weight_quant)
 *   y  [M, N] output, fp32 (y_dtype = FP8Q_OUT_F32) or bf16 bits (FP8Q_OUT_BF16, RNE of
 *      the fp32 accumulator). With K = 0 the output is all zeros.
 *   aq, wq, y: 16-byte aligned; sa, sw: 4-byte aligned. M, N >= 0 arbitrary (ragged tails
 *   are masked) up to 2^36 each, K a multiple of 128 and below 2^24 (at most 2^24 - 128).
 *   workspace / workspace_bytes: optional device scratch (16-byte aligned) for a split-K
 *   schedule, used by shapes with too few output tiles to fill the GPU; pass NULL / 0 to run
 *   without it. If workspace_bytes is smaller than fp8_block_gemm_workspace_bytes() the call
 *   runs without split-K (it does not fail). The workspace needs no initialisation: its
 *   arrival words are tagged with a per-launch epoch, so any contents, including those left
 *   by a call that never completed, count as no arrivals. Calls that may run at the same
 *   time must not share a workspace.
 *   The result does not depend on whether a workspace is given beyond fp32 rounding
 *   order (split-K sums the K ranges' fp32 partials in a fixed order), and is deterministic
 *   for a given (M, N, K, workspace size) call. */
int fp8_block_gemm(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw,
                   void *y, int y_dtype, int64_t M, int64_t N, int64_t K, void *workspace,
                   size_t workspace_bytes, void *stream);

/* fp8_block_gemm_bias -- fp8_block_gemm with a bias row added to the output.
 * (pomoai.com "DeepSeek-V3", the FP8 branch of linear(): y = fp8_gemm(...), then
 * y += bias when a bias is given.)
 *   bias [N] fp32 (4-byte aligned), or NULL for no bias. It is added to the fp32
 *   accumulator of every row before the output rounding, so a bf16 output is rounded once:
 *   Y[m, n] = RN_out(acc[m, n] + bias[n]).
 *   All other arguments, and the behaviour, are those of fp8_block_gemm (which is this
 *   call with bias = NULL). */
int fp8_block_gemm_bias(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw,
                        const float *bias, void *y, int y_dtype, int64_t M, int64_t N, int64_t K,
                        void *workspace, size_t workspace_bytes, void *stream);

/* fp8_bf16_gemm -- Y = X . W^T on bf16 operands: the bf16 branch of linear().
 * (pomoai.com "DeepSeek-V3", the linear() listing in section "FP8 mixed-precision
 * training": when the GEMM is not done in FP8, the weight is dequantised to bf16 by
 * weight_dequant and the layer is a plain bf16 linear, y = x . W^T, plus the bias.)
 *   x  [M, K] bf16 (bit patterns).              16-byte aligned.
 *   w  [N, K] bf16, e.g. from fp8_weight_dequant. 16-byte aligned.
 *   bias [N] fp32 or NULL; added to the fp32 accumulator before the output rounding.
 *                                               4-byte aligned.
 *   y  [M, N]: fp32 (y_dtype = FP8Q_OUT_F32) or bf16 bits (FP8Q_OUT_BF16, RNE of the fp32
 *      accumulator).                            4-byte aligned.
 *   Every product is exact in fp32; the products are summed in fp32 by the bf16 matrix
 *   unit, 32 at a time, the partial sums chained in fp32 along K. M, N >= 0 arbitrary
 *   (ragged tails masked), M and N up to 2^36; K a multiple of 64 below 2^23 (FP8Q_ERR_SHAPE
 *   otherwise). With K = 0 the output is the bias (or zeros). */
int fp8_bf16_gemm(const uint16_t *x, const uint16_t *w, const float *bias, void *y, int y_dtype,
                  int64_t M, int64_t N, int64_t K, void *stream);

/* fp8_block_gemm_noalloc -- fp8_block_gemm for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). It
 * calls no allocating routine; in place of the workspace argument it uses a static split-K
 * scratch of FP8Q_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, which the library holds on every
 * GPU it is loaded on until the process ends.
 *   Arguments, layouts, modes (y_dtype), alignment and results: as fp8_block_gemm, whose
 *   tile and split-K plan it uses, so its output is bit-identical to fp8_block_gemm's with a
 *   workspace of fp8_block_gemm_workspace_bytes() bytes.
 *   Returns FP8Q_ERR_WORKSPACE, enqueueing nothing, when fp8_block_gemm_workspace_bytes()
 *   for the shape and y_dtype exceeds FP8Q_NOALLOC_SCRATCH_BYTES.
 *   The scratch needs no clearing (its split-K arrival words are tagged per launch) and keeps
 *   the last call's contents. Every call on one GPU shares that GPU's scratch: calls that may
 *   overlap on one GPU (other streams, other host threads) race and must be serialised by the
 *   caller. */
#define FP8Q_NOALLOC_SCRATCH_BYTES ((size_t)33554432)
int fp8_block_gemm_noalloc(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw,
                           void *y, int y_dtype, int64_t M, int64_t N, int64_t K, void *stream);

/* fp8_grouped_gemm -- the block-scaled GEMMs of several experts in one launch, for the
 * routed experts of a mixture-of-experts layer: expert e multiplies its own rows of A by its
 * own FP8 weight. (pomoai.com "DeepSeek-V3", MoE section: each token is routed to 8 of
 * 256 experts; FP8 section: every expert weight is stored as E4M3 128x128 blocks.)
 *   aq [rows, K] E4M3 and sa [rows, K/128] fp32: the activation rows of all experts, those
 *      of expert e contiguous (layout of fp8_act_quant).
 *   wq [experts, N, K] E4M3 and sw [experts, ceil(N/128), K/128] fp32: expert e's weight
 *      and scales (layout of fp8_weight_quant, one after another).
 *   offsets: DEVICE int64 [experts + 1]; expert e owns rows [offsets[e], offsets[e+1]).
 *      Expected 0 = offsets[0] <= offsets[1] <= ... <= offsets[experts] <= rows. Each
 *      expert's range is clamped to [0, rows] (an empty range where offsets[e+1] <
 *      offsets[e]), so nothing is read or written outside the buffers whatever the values;
 *      ranges that overlap after clamping write their common rows more than once, in an
 *      unspecified order. 8-byte aligned; read by the kernel, so it may be produced by
 *      earlier work on the same stream.
 *   y [rows, N]: row r is the output of the expert that owns it; rows owned by no expert
 *      are not written. y_dtype as for fp8_block_gemm (output dtype and contraction mode).
 *   1 <= experts <= 1024. No split-K, no workspace. Other conventions as fp8_block_gemm. */
int fp8_grouped_gemm(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw,
                     const int64_t *offsets, void *y, int y_dtype, int64_t experts, int64_t rows,
                     int64_t N, int64_t K, void *stream);

/* ---- Training GEMMs (backward of linear()) -------------------------------------------
 * The pages train in FP8 with E4M3 everywhere (88811315.cn post 75335, Float8-training
 * paragraph; pomoai.com "DeepSeek-V3", "FP8 mixed-precision training") but give the
 * backward pass's granularity nowhere. Reading taken here: each GEMM operand is quantised
 * by the forward rules along its contraction dimension. For y = x W^T:
 *   activation gradient dX [M, K] = dY [M, N] . W [N, K]: dY by fp8_act_quant (1x128 tiles
 *     along N); W's 128x128 blocks are square, so W^T has the same codes and block scales,
 *     transposed (fp8_weight_transpose), and dX = fp8_block_gemm(dYq, sdy, Wq^T, sw^T).
 *   weight gradient dW [N, K] = dY^T . X, contracted over tokens: dY and X both quantised in
 *     1x128 tiles along the token dimension (fp8_act_quant_t), and
 *     dW = fp8_rowwise_gemm(dY^T q, s, X^T q, s) with per-row scales on both operands. */

/* fp8_act_quant_t -- token-wise quantisation with a transposed output.
 *   x [M, C] bf16 (row-major; C a multiple of 8).
 *   qt [C, ldq] E4M3 and st [C, ldq/128] fp32, ldq = ceil(M/128)*128: row c holds channel c
 *      over all tokens; the tile (c, mb) covers tokens 128 mb .. 128 mb + 127 and follows
 *      fp8_act_quant's rules (amax over the tile, s = RN(amax/448), RNE-saturated codes).
 *      Tokens M .. ldq-1 are written as code 0 and enter no amax, so qt can be contracted
 *      over ldq directly.
 *   Alignment: x, qt 16 bytes; st 4. M or C = 0: no-op. */
int fp8_act_quant_t(const uint16_t *x, uint8_t *qt, float *st, int64_t M, int64_t C, void *stream);

/* fp8_weight_transpose -- Wq [N, K] E4M3 -> Wq^T [K, N]; sw [ceil(N/128), K/128] ->
 *   sw^T [K/128, ceil(N/128)]. K a multiple of 128; any N >= 0 (a contraction over N in a
 *   block GEMM needs N to be a multiple of 128). wq, wqt 16-byte aligned; sw, swt 4. */
int fp8_weight_transpose(const uint8_t *wq, const float *sw, uint8_t *wqt, float *swt, int64_t N, int64_t K,
                         void *stream);

/* fp8_rowwise_gemm -- Y [M, N] = sum over slices kb of P[m,n,kb] * sa[m,kb] * sb[n,kb],
 *   P the exact contraction of 128-wide K slice kb of aq [M, K] and bq [N, K] (both E4M3,
 *   K-contiguous), sa [M, K/128], sb [N, K/128] fp32: fp8_block_gemm with a per-row scale on
 *   the second operand instead of a 128x128 block scale. y_dtype, modes, workspace (size from
 *   fp8_rowwise_gemm_workspace_bytes), alignment and errors as for fp8_block_gemm; no bias. */
int fp8_rowwise_gemm(const uint8_t *aq, const float *sa, const uint8_t *bq, const float *sb, void *y, int y_dtype,
                     int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes, void *stream);
size_t fp8_rowwise_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int y_dtype);

/* Workspace size in bytes that lets fp8_block_gemm use its split-K schedule for this
 * shape and y_dtype (including the mode bits); 0 if that call does not use one or the
 * arguments are invalid. Host-only; enqueues nothing. */
size_t fp8_block_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int y_dtype);

/* Tuning and test hook (not needed for normal use). fp8_block_gemm normally picks its tile
 * configuration and split-K count per shape from a cost model fitted to MI355X timings.
 * fp8q_gemm_force_config(config, splits) makes every later call in the process use tile
 * configuration `config` (0 <= config < number of configurations; -1 restores the
 * automatic choice) and `splits` K ranges (1..8 when the shape and workspace allow it;
 * 0 restores the automatic choice). A configuration the contraction mode does not
 * implement falls back to its default configuration. Returns FP8Q_ERR_SHAPE for values out
 * of range. Process-wide and not synchronised with calls in flight on other threads.
 * fp8q_gemm_config_name(config) names a configuration ("256x256w8": BM x BN, w8 = 8
 * waves, s2 = two stages), or returns NULL past the last one.
 * fp8q_gemm_plan(M, N, K, y_dtype, &config, &splits) reports the configuration and split count
 * fp8_block_gemm would use for that shape and y_dtype (the same flags) when given a workspace
 * of at least fp8_block_gemm_workspace_bytes, forced choices included. Returns FP8Q_OK, or
 * FP8Q_ERR_NULL / FP8Q_ERR_DTYPE / FP8Q_ERR_SHAPE (M, N, K must be positive) without writing
 * the outputs. */
/* The same choice can be made for a whole process through the environment, read once at
 * the first GEMM call: FP8Q_GEMM_TILE=<configuration name> and FP8Q_GEMM_SPLITS=<count>.
 * FP8Q_AQ_WGS_PER_CU=<1..32> sets fp8_act_quant's resident workgroups per CU (default 16).
 * FP8Q_BF16_TILE=256x256, 128x128 or 64x128 pins fp8_bf16_gemm's tile (read at every call;
 * by default chosen from the shape). */
int fp8q_gemm_force_config(int config, int splits);
const char *fp8q_gemm_config_name(int config);
int fp8q_gemm_plan(int64_t M, int64_t N, int64_t K, int y_dtype, int *config, int *splits);

/* Static string describing a status code (never NULL). */
const char *fp8q_strerror(int status);

/* Library ABI version, (major << 16) | minor. */
int fp8q_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
