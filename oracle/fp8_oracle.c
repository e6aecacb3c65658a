/*
 * fp8_oracle.c -- plain CPU reference for FP8 (E4M3) fine-grained block quantisation
 * and the block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE. This file is the checker, not the product: only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load or call it. It shares no
 * code, header, table or constant with the GPU library, and never includes it.
 *
 * Written from these pages (cited by title and section):
 *   [P1] 88811315.cn post 75335 (essay on DeepSeek v3), the Float8-training paragraph:
 *        E4M3 is used for every GEMM operand, and FP8 partial products are promoted into
 *        a high-precision FP32 accumulator.
 *   [P4] qdgithub.com book 25/317, section "FP8 quantisation: balancing storage and
 *        compute": matrices are split into row/column blocks, FP8 is used inside a block
 *        and dequantisation happens outside the matrix units.
 *   [P5] pomoai.com hub page "DeepSeek-V3", section "FP8 mixed-precision training":
 *        float8 e4m3; weights in 128x128 blocks, one float32 scale per block
 *        (weight_scale_inv); activations quantised at run time per token per 128
 *        channels; and the linear() listing in that section, which returns the GEMM
 *        output without re-quantising it.
 * Constants the pages leave open are fixed as: OCP E4M3FN (bias 7, largest finite 448,
 * S.1111.111 is NaN, no infinities), scale = amax / 448 as an IEEE fp32 division,
 * element code = E4M3 round-to-nearest-even with saturation of RN_fp32(x / scale).
 *
 * Floating point: build with -ffp-contract=off and without -ffast-math; every fp32
 * operation here is a single IEEE-754 operation rounded to nearest-even, and every
 * float64 sum of E4M3 products is exact (see or_block_gemm).
 *
 * The OpenMP pragmas only split independent rows/blocks across threads; they do not
 * change any arithmetic or its order.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_BLOCK 128

/* ---------------------------------------------------------------------------------
 * Scalar codecs
 * ------------------------------------------------------------------------------- */

/* bf16 is the upper half of an IEEE binary32, so widening is exact. */
float or_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Value of a bf16 bit pattern in float64, treating 0x7F80 (the pattern after the
 * largest finite value) as 2^128 so that it can serve as the upper neighbour of the
 * largest finite value when rounding. */
static double bf16_as_double_ext(uint16_t b)
{
    if ((b & 0x7FFF) == 0x7F80)
        return (b & 0x8000) ? -ldexp(1.0, 128) : ldexp(1.0, 128);
    return (double)or_bf16_to_f32(b);
}

/* Round an fp32 value to the nearest bf16 (8 significant bits), ties to the pattern
 * with an even last bit; above the largest finite value by half an ulp or more gives
 * infinity. Written as "pick the nearer of the two bf16 values that bracket v":
 * the truncated pattern and its successor in magnitude. Both distances are exact in
 * float64 (v has 24 significant bits and the candidates lie in v's binade or at its
 * upper edge). */
uint16_t or_f32_to_bf16(float v)
{
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    if (isnan(v))
        return (uint16_t)((u >> 16) | 0x0040);
    uint16_t lo = (uint16_t)(u >> 16);     /* |lo| <= |v| */
    if ((uint32_t)lo << 16 == u)
        return lo;                           /* exactly representable */
    uint16_t hi = (uint16_t)(lo + 1);      /* next pattern away from zero */
    double dv = (double)v;
    double dlo = fabs(dv - bf16_as_double_ext(lo));
    double dhi = fabs(bf16_as_double_ext(hi) - dv);
    if (dlo < dhi)
        return lo;
    if (dhi < dlo)
        return hi;
    return (lo & 1) ? hi : lo;
}

/* Round a float64 value to the nearest bf16, ties to the even pattern, by the same
 * "nearer of the two bracketing bf16 values" rule. The lower candidate is the bf16
 * truncation (toward zero) of the fp32 truncation of v, so |lo| <= |v| < |lo + 1|; both
 * distances are exact in float64 (Sterbenz: the candidates lie within a factor of two
 * of v). Used for the rounded reference of bf16 GEMM outputs. */
uint16_t or_f64_to_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    float f = (float)v;
    if (fabs((double)f) > fabs(v))
        f = nextafterf(f, 0.0f);          /* truncate toward zero */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t lo = (uint16_t)(u >> 16);
    if ((lo & 0x7FFF) >= 0x7F80)
        return lo;                         /* |v| beyond every finite fp32: infinity */
    if (bf16_as_double_ext(lo) == v)
        return lo;
    uint16_t hi = (uint16_t)(lo + 1);
    double dlo = fabs(v - bf16_as_double_ext(lo));
    double dhi = fabs(bf16_as_double_ext(hi) - v);
    if (dlo < dhi)
        return lo;
    if (dhi < dlo)
        return hi;
    return (lo & 1) ? hi : lo;
}

/* OCP E4M3FN decode, closed form. Code s.eeee.mmm:
 *   e = 15 and m = 7 -> NaN;  e = 0 -> m * 2^-9 (subnormal);  else (8 + m) * 2^(e - 10),
 * i.e. (1 + m/8) * 2^(e - 7) with exponent bias 7; the sign is applied last. */
double or_e4m3_decode(uint8_t b)
{
    int sign = b >> 7;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = (double)m * ldexp(1.0, -9);
    else
        v = (double)(8 + m) * ldexp(1.0, e - 10);
    return sign ? -v : v;
}

/* Values of all 256 codes, filled once at load time from the closed-form decoder. */
static double e4m3_value[256];

__attribute__((constructor)) static void fill_e4m3_values(void)
{
    for (int c = 0; c < 256; ++c)
        e4m3_value[c] = or_e4m3_decode((uint8_t)c);
}

/* OCP E4M3FN encode with round-to-nearest-even and saturation.
 * NaN -> 0x7F | sign; |v| >= 448 -> 0x7E | sign (largest finite, never NaN).
 * Otherwise the code is found by searching all 127 non-negative finite E4M3 values
 * (codes 0x00..0x7E, from the closed-form decoder) for the one nearest to |v|; on an
 * exact tie the even code (mantissa LSB 0) wins. The sign bit of v is then OR-ed in, so
 * a negative value that rounds to zero gives 0x80.
 * The two nearest candidates bracket |v| within a factor of two (or one of them is 0),
 * so their distances to |v| are exact in float64; farther candidates can only be
 * farther after rounding. */
uint8_t or_e4m3_encode(float v)
{
    if (isnan(v))
        return signbit(v) ? 0xFF : 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    int best = 0;
    double bestd = a; /* distance to code 0x00 (value 0) */
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(a - e4m3_value[c]);
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)(sign | best);
}

/* ---------------------------------------------------------------------------------
 * Quantisation of one group of values sharing one scale. The group is given as a list
 * of pointers-with-stride so that a 1x128 activation tile and a (<=128)x128 weight block
 * use the same steps:
 *   amax  = max |x|                                     (exact)
 *   scale = RN_fp32(amax / 448)                         (IEEE fp32 division)
 *   div   = scale, or 1 when amax == 0                  (all-zero group: codes are +-0)
 *   code  = E4M3_RNE_SAT(RN_fp32(x / div))              (IEEE fp32 division, then encode)
 * ------------------------------------------------------------------------------- */
static float quant_group(const uint16_t *x, int64_t rows, int64_t row_stride, int64_t cols,
                         uint8_t *q, int64_t q_stride)
{
    float amax = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float a = fabsf(or_bf16_to_f32(x[r * row_stride + c]));
            if (a > amax)
                amax = a;
        }
    float scale = amax / 448.0f;
    float div = (amax == 0.0f) ? 1.0f : scale;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            q[r * q_stride + c] = or_e4m3_encode(or_bf16_to_f32(x[r * row_stride + c]) / div);
    return scale;
}

/* Activation quantisation, per token per 128 channels ([P5] FP8 section: dynamic
 * activation quantisation at per-token-per-128-channel granularity).
 * x: bf16 [M, K] row-major; q: E4M3 [M, K]; s: fp32 [M, K/128] row-major,
 * s[m, kb] is the scale of tile x[m, 128*kb : 128*kb + 128]. K must be a multiple of 128. */
void or_act_quant(const uint16_t *x, uint8_t *q, float *s, int64_t M, int64_t K)
{
    int64_t nkb = K / OR_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t kb = 0; kb < nkb; ++kb)
            s[m * nkb + kb] = quant_group(x + m * K + kb * OR_BLOCK, 1, K, OR_BLOCK,
                                          q + m * K + kb * OR_BLOCK, K);
}

/* Weight quantisation in 128x128 blocks ([P5] FP8 section: FP8 weights stored in 128x128
 * blocks, each with its own float32 scale factor weight_scale_inv).
 * w: bf16 [N, K]; q: E4M3 [N, K]; s: fp32 [ceil(N/128), K/128] row-major. The last
 * block row covers rows [128*nb, N) only, so its amax is over the valid rows. */
void or_weight_quant(const uint16_t *w, uint8_t *q, float *s, int64_t N, int64_t K)
{
    int64_t nkb = K / OR_BLOCK;
    int64_t nnb = (N + OR_BLOCK - 1) / OR_BLOCK;
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t nb = 0; nb < nnb; ++nb)
        for (int64_t kb = 0; kb < nkb; ++kb) {
            int64_t r0 = nb * OR_BLOCK;
            int64_t rows = (N - r0 < OR_BLOCK) ? (N - r0) : OR_BLOCK;
            s[nb * nkb + kb] = quant_group(w + r0 * K + kb * OR_BLOCK, rows, K, OR_BLOCK,
                                           q + r0 * K + kb * OR_BLOCK, K);
        }
}

/* Weight dequantisation ([P5] FP8 section, the bf16 branch of linear(): the FP8 weight
 * and its scale are turned back into a high-precision weight; [P4]: dequantisation
 * outside the matrix units). Each element: RN_bf16(RN_fp32(decode(q) * s[n/128, k/128])).
 * decode(q) is exactly representable in fp32, so the product is one fp32 rounding. */
void or_weight_dequant(const uint8_t *q, const float *s, uint16_t *w, int64_t N, int64_t K)
{
    int64_t nkb = K / OR_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)or_e4m3_decode(q[n * K + k]);
            float p = v * s[(n / OR_BLOCK) * nkb + k / OR_BLOCK];
            w[n * K + k] = or_f32_to_bf16(p);
        }
}

/* ---------------------------------------------------------------------------------
 * Block-scaled GEMM, Y = A . W^T ([P4]: FP8 products inside a block, dequantisation
 * outside; [P1]: FP8 partials promoted into an FP32 main accumulator; [P5] linear():
 * fp8_gemm(x, scale, weight, weight.scale), output not re-quantised).
 * For output (m, n), with slices kb = 0 .. K/128 - 1:
 *   P_kb  = sum_{k in slice kb} decode(aq[m,k]) * decode(wq[n,k])
 *   f_kb  = sa[m, kb] * sw[n/128, kb]
 *   y     = sum_kb P_kb * f_kb
 *   bound = sum_kb (sum_{k in slice} |decode(aq[m,k]) * decode(wq[n,k])|) * |f_kb|
 *         = sum_k |a_k * w_k| over the dequantised operands.
 * Exactness: each E4M3 value is an integer multiple of 2^-9 with magnitude <= 448, so
 * every product is a multiple of 2^-18 below 2^18 and every slice partial (128 terms)
 * needs at most 44 significant bits: P_kb is exact in float64 in any order. f_kb is the
 * exact product of two fp32 values (48 bits). The only float64 roundings are P_kb*f_kb
 * and the sum over slices, so y is the method's exact result up to ~1e-15 * bound.
 * ------------------------------------------------------------------------------- */
static void gemm_one(const double *dec, const uint8_t *aq, const float *sa, const uint8_t *wq,
                     const float *sw, int64_t N, int64_t K, int64_t m, int64_t n,
                     double *y_out, double *bound_out)
{
    (void)N;
    int64_t nkb = K / OR_BLOCK;
    const uint8_t *arow = aq + m * K;
    const uint8_t *wrow = wq + n * K;
    double y = 0.0, bound = 0.0;
    for (int64_t kb = 0; kb < nkb; ++kb) {
        double p = 0.0, pabs = 0.0;
        for (int64_t k = kb * OR_BLOCK; k < (kb + 1) * OR_BLOCK; ++k) {
            double t = dec[arow[k]] * dec[wrow[k]];
            p += t;
            pabs += fabs(t);
        }
        double f = (double)sa[m * nkb + kb] * (double)sw[(n / OR_BLOCK) * nkb + kb];
        y += p * f;
        bound += pabs * fabs(f);
    }
    *y_out = y;
    *bound_out = bound;
}

/* Full output: y and bound are float64 [M, N] row-major. */
void or_block_gemm(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw,
                   int64_t M, int64_t N, int64_t K, double *y, double *bound)
{
    const double *dec = e4m3_value;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            gemm_one(dec, aq, sa, wq, sw, N, K, m, n, y + m * N + n, bound + m * N + n);
}

/* Sampled outputs: for i < count, y[i], bound[i] are output (rows[i], cols[i]). */
void or_block_gemm_sampled(const uint8_t *aq, const float *sa, const uint8_t *wq,
                           const float *sw, int64_t M, int64_t N, int64_t K,
                           const int64_t *rows, const int64_t *cols, int64_t count, double *y,
                           double *bound)
{
    (void)M;
    const double *dec = e4m3_value;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i)
        gemm_one(dec, aq, sa, wq, sw, N, K, rows[i], cols[i], y + i, bound + i);
}

/* ---------------------------------------------------------------------------------
 * GEMM with per-row scales on both operands (the weight-gradient reading: both operands
 * quantised in 1x128 tiles along the contraction dimension). For output (m, n):
 *   P_kb = sum_{k in slice kb} decode(aq[m,k]) * decode(bq[n,k])   (exact, as above)
 *   y    = sum_kb P_kb * (sa[m, kb] * sb[n, kb]),  bound = sum_kb |P|_kb * |sa * sb|.
 * With sb rows equal within each 128-row block this is or_block_gemm.
 * ------------------------------------------------------------------------------- */
static void rowwise_one(const double *dec, const uint8_t *aq, const float *sa, const uint8_t *bq,
                        const float *sb, int64_t K, int64_t m, int64_t n, double *y_out,
                        double *bound_out)
{
    int64_t nkb = K / OR_BLOCK;
    const uint8_t *arow = aq + m * K;
    const uint8_t *brow = bq + n * K;
    double y = 0.0, bound = 0.0;
    for (int64_t kb = 0; kb < nkb; ++kb) {
        double p = 0.0, pabs = 0.0;
        for (int64_t k = kb * OR_BLOCK; k < (kb + 1) * OR_BLOCK; ++k) {
            double t = dec[arow[k]] * dec[brow[k]];
            p += t;
            pabs += fabs(t);
        }
        double f = (double)sa[m * nkb + kb] * (double)sb[n * nkb + kb];
        y += p * f;
        bound += pabs * fabs(f);
    }
    *y_out = y;
    *bound_out = bound;
}

void or_rowwise_gemm(const uint8_t *aq, const float *sa, const uint8_t *bq, const float *sb,
                     int64_t M, int64_t N, int64_t K, double *y, double *bound)
{
    const double *dec = e4m3_value;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            rowwise_one(dec, aq, sa, bq, sb, K, m, n, y + m * N + n, bound + m * N + n);
}

void or_rowwise_gemm_sampled(const uint8_t *aq, const float *sa, const uint8_t *bq,
                             const float *sb, int64_t K, const int64_t *rows,
                             const int64_t *cols, int64_t count, double *y, double *bound)
{
    const double *dec = e4m3_value;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i)
        rowwise_one(dec, aq, sa, bq, sb, K, rows[i], cols[i], y + i, bound + i);
}

/* ---------------------------------------------------------------------------------
 * bf16 linear (the linear() listing's bf16 branch, [P5]: the FP8 weight is dequantised by
 * weight_dequant and the layer is a plain bf16 linear y = x . W^T):
 *   y[m, n]     = sum_k x[m, k] * w[n, k]
 *   bound[m, n] = sum_k |x[m, k] * w[n, k]|
 * over the bf16 values (x and the dequantised w), in float64. Each bf16 x bf16 product is
 * exact in float64 (16 significant bits); the float64 sum rounds at ~2^-53 relative to
 * the bound, far below the fp32 accumulation it checks.
 * ------------------------------------------------------------------------------- */
void or_matmul_bf16(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N, int64_t K, double *y,
                    double *bound)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const uint16_t *wr = w + n * K;
            double acc = 0.0, b = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double t = (double)or_bf16_to_f32(xr[k]) * (double)or_bf16_to_f32(wr[k]);
                acc += t;
                b += fabs(t);
            }
            y[m * N + n] = acc;
            bound[m * N + n] = b;
        }
    }
}

/* Unquantised float64 product of the original bf16 operands at sampled outputs, for the
 * informational relative error of the FP8 path: y[i] = sum_k x[r,k] * w[c,k]. */
void or_matmul_bf16_sampled(const uint16_t *x, const uint16_t *w, int64_t K, const int64_t *rows,
                            const int64_t *cols, int64_t count, double *y)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        const uint16_t *xr = x + rows[i] * K;
        const uint16_t *wr = w + cols[i] * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += (double)or_bf16_to_f32(xr[k]) * (double)or_bf16_to_f32(wr[k]);
        y[i] = acc;
    }
}

/* ---------------------------------------------------------------------------------
 * Batch helpers for tests (vectorised calls of the scalar codecs above).
 * ------------------------------------------------------------------------------- */
void or_e4m3_encode_batch(const float *v, uint8_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_e4m3_encode(v[i]);
}

void or_f32_to_bf16_batch(const float *v, uint16_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_f32_to_bf16(v[i]);
}

void or_f64_to_bf16_batch(const double *v, uint16_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_f64_to_bf16(v[i]);
}

int or_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void or_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
