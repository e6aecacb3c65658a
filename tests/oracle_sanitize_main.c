/*
 * oracle_sanitize_main.c -- drives every entry point of the CPU oracle (oracle/fp8_oracle.c)
 * on small ragged inputs, built with AddressSanitizer and UndefinedBehaviorSanitizer, so
 * that an out-of-bounds access, overflow or other undefined behaviour in the checker
 * aborts the run. Every buffer is allocated at exactly its size. A few invariants are
 * checked on the way so that the run also exercises real values:
 *   decode(encode(decode(c))) == decode(c) for every finite code;
 *   every act_quant / weight_quant code is finite and re-encodes to itself;
 *   block_gemm and block_gemm_sampled agree bit for bit;
 *   the bound is at least |y|.
 * Test infrastructure only (built and run by tests/test_oracle_sanitize.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float or_bf16_to_f32(uint16_t b);
uint16_t or_f32_to_bf16(float v);
uint16_t or_f64_to_bf16(double v);
double or_e4m3_decode(uint8_t b);
uint8_t or_e4m3_encode(float v);
void or_act_quant(const uint16_t *x, uint8_t *q, float *s, int64_t M, int64_t K);
void or_weight_quant(const uint16_t *w, uint8_t *q, float *s, int64_t N, int64_t K);
void or_weight_dequant(const uint8_t *q, const float *s, uint16_t *w, int64_t N, int64_t K);
void or_block_gemm(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw, int64_t M, int64_t N,
                   int64_t K, double *y, double *bound);
void or_block_gemm_sampled(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw, int64_t M,
                           int64_t N, int64_t K, const int64_t *rows, const int64_t *cols, int64_t n, double *y,
                           double *bound);
void or_rowwise_gemm(const uint8_t *aq, const float *sa, const uint8_t *bq, const float *sb, int64_t M, int64_t N,
                     int64_t K, double *y, double *bound);
void or_rowwise_gemm_sampled(const uint8_t *aq, const float *sa, const uint8_t *bq, const float *sb, int64_t K,
                             const int64_t *rows, const int64_t *cols, int64_t n, double *y, double *bound);
void or_matmul_bf16_sampled(const uint16_t *x, const uint16_t *w, int64_t K, const int64_t *rows, const int64_t *cols,
                            int64_t n, double *y);
void or_matmul_bf16(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N, int64_t K, double *y, double *bound);
void or_e4m3_encode_batch(const float *v, uint8_t *out, int64_t n);
void or_f32_to_bf16_batch(const float *v, uint16_t *out, int64_t n);
void or_f64_to_bf16_batch(const double *v, uint16_t *out, int64_t n);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {   /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

/* random finite bf16 patterns of varied magnitude, some zero tiles and subnormals */
static void fill_bf16(uint16_t *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = next_u64();
        uint16_t exp = (uint16_t)(100 + (r % 60));          /* 2^-27 .. 2^32 */
        uint16_t v = (uint16_t)(((r >> 8) & 0x8000) | (exp << 7) | ((r >> 20) & 0x7F));
        if ((r >> 40) % 17 == 0) v = (uint16_t)((r >> 44) & 0x807F);   /* zero or subnormal */
        x[i] = v;
    }
}

static int fail(const char *what) {
    fprintf(stderr, "invariant failed: %s\n", what);
    return 1;
}

int main(void) {
    /* codecs */
    for (int c = 0; c < 256; ++c) {
        if ((c & 0x7F) == 0x7F) continue;
        double v = or_e4m3_decode((uint8_t)c);
        if (or_e4m3_decode(or_e4m3_encode((float)v)) != v) return fail("decode(encode(decode(c)))");
    }
    float fv[7] = {0.0f, -0.0f, 448.0f, 1e30f, -1e-30f, 3.0f * 0.0009765625f, NAN};
    uint8_t fq[7];
    or_e4m3_encode_batch(fv, fq, 7);
    uint16_t fb[7];
    or_f32_to_bf16_batch(fv, fb, 7);
    double dv[3] = {1.0 + 1e-9, -3.5e38, 1e-45};
    uint16_t db[3];
    or_f64_to_bf16_batch(dv, db, 3);

    const int64_t M = 37, N = 300, K = 384, nkb = K / 128, nnb = (N + 127) / 128;
    uint16_t *x = xmalloc(sizeof(uint16_t) * M * K), *w = xmalloc(sizeof(uint16_t) * N * K);
    fill_bf16(x, M * K);
    fill_bf16(w, N * K);
    for (int64_t k = 0; k < 128; ++k) x[3 * K + 128 + k] = 0;   /* an all-zero tile */
    uint8_t *aq = xmalloc((size_t)M * K), *wq = xmalloc((size_t)N * K), *bq = xmalloc((size_t)N * K);
    float *sa = xmalloc(sizeof(float) * M * nkb), *sw = xmalloc(sizeof(float) * nnb * nkb);
    float *sb = xmalloc(sizeof(float) * N * nkb);
    or_act_quant(x, aq, sa, M, K);
    or_weight_quant(w, wq, sw, N, K);
    or_act_quant(w, bq, sb, N, K);     /* per-row scales on the second operand */
    for (int64_t i = 0; i < M * K; ++i)
        if ((aq[i] & 0x7F) == 0x7F || or_e4m3_encode((float)or_e4m3_decode(aq[i])) != aq[i]) return fail("act code");
    for (int64_t i = 0; i < N * K; ++i)
        if ((wq[i] & 0x7F) == 0x7F) return fail("weight code");
    uint16_t *wd = xmalloc(sizeof(uint16_t) * N * K);
    or_weight_dequant(wq, sw, wd, N, K);

    double *y = xmalloc(sizeof(double) * M * N), *b = xmalloc(sizeof(double) * M * N);
    or_block_gemm(aq, sa, wq, sw, M, N, K, y, b);
    const int64_t S = 64;
    int64_t *rows = xmalloc(sizeof(int64_t) * S), *cols = xmalloc(sizeof(int64_t) * S);
    for (int64_t i = 0; i < S; ++i) {
        rows[i] = (int64_t)(next_u64() % (uint64_t)M);
        cols[i] = (int64_t)(next_u64() % (uint64_t)N);
    }
    rows[0] = M - 1;
    cols[0] = N - 1;
    double *ys = xmalloc(sizeof(double) * S), *bs = xmalloc(sizeof(double) * S);
    or_block_gemm_sampled(aq, sa, wq, sw, M, N, K, rows, cols, S, ys, bs);
    for (int64_t i = 0; i < S; ++i) {
        double yf = y[rows[i] * N + cols[i]], bf = b[rows[i] * N + cols[i]];
        if (memcmp(&yf, &ys[i], sizeof yf) != 0 || memcmp(&bf, &bs[i], sizeof bf) != 0) return fail("sampled == full");
    }
    for (int64_t i = 0; i < M * N; ++i)
        if (!(b[i] >= fabs(y[i]) * (1.0 - 1e-12))) return fail("bound >= |y|");
    or_rowwise_gemm(aq, sa, bq, sb, M, N, K, y, b);
    or_rowwise_gemm_sampled(aq, sa, bq, sb, K, rows, cols, S, ys, bs);
    for (int64_t i = 0; i < S; ++i)
        if (y[rows[i] * N + cols[i]] != ys[i]) return fail("rowwise sampled == full");
    or_matmul_bf16_sampled(x, w, K, rows, cols, S, ys);
    or_matmul_bf16(x, wd, M, N, K, y, b);
    or_matmul_bf16_sampled(x, wd, K, rows, cols, S, bs);
    for (int64_t i = 0; i < S; ++i)
        if (y[rows[i] * N + cols[i]] != bs[i]) return fail("bf16 matmul sampled == full");

    free(x); free(w); free(aq); free(wq); free(bq); free(sa); free(sw); free(sb); free(wd);
    free(y); free(b); free(rows); free(cols); free(ys); free(bs);
    printf("oracle sanitize: ok\n");
    return 0;
}
