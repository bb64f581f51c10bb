/*
 * Driver for the address / undefined-behaviour sanitizer build of the CPU
 * oracle (test infrastructure): every oracle function on small seeded inputs,
 * including all-zero, subnormal and near-overflow groups and ragged row
 * lists, with buffers of exactly the documented sizes so that any access past
 * them is reported.  Exit status 0 when every call ran and the few
 * self-consistency checks hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e4m3_decode(uint8_t c);
uint8_t oracle_e4m3_encode(double v);
void oracle_quant_act(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s);
void oracle_quant_wblock(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s);
void oracle_prune24_mask(const uint16_t *w, const float *c, int64_t N, int64_t K, uint8_t *keep);
void oracle_prune24_compress(const uint16_t *w, const float *c, int64_t N, int64_t K, uint8_t *vals, uint8_t *meta,
                             float *s);
void oracle_prune24_compress_tensor(const uint16_t *w, const float *c, int64_t N, int64_t K, uint8_t *vals,
                                    uint8_t *meta, float *s);
void oracle_decompress24(const uint8_t *vals, const uint8_t *meta, int64_t N, int64_t K, uint8_t *q);
void oracle_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws, int64_t M, int64_t N,
                 int64_t K, double *y);
void oracle_gemm_rows(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws, int64_t M, int64_t N,
                      int64_t K, const int64_t *rows, int64_t R, double *y);
void oracle_quant_act_static(const uint16_t *x, int64_t M, int64_t K, float s_in, uint8_t *q, float *s);
void oracle_quant_act_tensor(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s);
void oracle_quant_act_ue8m0(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, uint8_t *e);
void oracle_quant_wblock_ue8m0(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, uint8_t *e);
int oracle_num_threads(void);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {  /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

/* finite bf16 bit patterns of every exponent, zeros and subnormals included */
static uint16_t rnd_bf16(void) {
    uint16_t b;
    do b = (uint16_t)rnd(); while (((b >> 7) & 0xFF) == 0xFF);
    return b;
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

static int fail(const char *what) {
    fprintf(stderr, "check failed: %s\n", what);
    return 1;
}

static int run_shape(int64_t M, int64_t N, int64_t K) {
    int bad = 0;
    uint16_t *x = xmalloc((size_t)(M * K) * 2), *w = xmalloc((size_t)(N * K) * 2);
    float *c = xmalloc((size_t)K * 4);
    for (int64_t i = 0; i < M * K; i++) x[i] = rnd_bf16();
    for (int64_t i = 0; i < N * K; i++) w[i] = rnd_bf16();
    for (int64_t k = 0; k < K; k++) c[k] = (float)(rnd() % 7);  /* zero and equal norms */
    /* special groups: all zero, all negative zero, one subnormal */
    for (int64_t k = 0; k < 128 && k < K; k++) { x[k] = 0; w[k] = 0x8000; }
    if (M > 1) for (int64_t k = 0; k < 128; k++) x[K + k] = 1;
    uint8_t *xq = xmalloc((size_t)(M * K)), *wq = xmalloc((size_t)(N * K)), *keep = xmalloc((size_t)(N * K));
    float *xs = xmalloc((size_t)(M * (K / 128)) * 4), *ws = xmalloc((size_t)((N / 128) * (K / 128)) * 4);
    uint8_t *xe = xmalloc((size_t)(M * (K / 128))), *we = xmalloc((size_t)((N / 128) * (K / 128)));
    uint8_t *vals = xmalloc((size_t)(N * K / 2)), *meta = xmalloc((size_t)(N * K / 8));
    uint8_t *dq = xmalloc((size_t)(N * K));
    float *s2 = xmalloc((size_t)((N / 128) * (K / 128)) * 4);
    double *y = xmalloc((size_t)(M * N) * 8), *yr = xmalloc((size_t)(3 * N) * 8);

    oracle_quant_act(x, M, K, xq, xs);
    oracle_quant_wblock(w, N, K, wq, ws);
    oracle_quant_act_ue8m0(x, M, K, xq, xe);
    oracle_quant_wblock_ue8m0(w, N, K, wq, we);
    oracle_quant_act_tensor(x, M, K, xq, xs);
    oracle_quant_act_static(x, M, K, 0.5f, xq, xs);
    for (int pass = 0; pass < 2; pass++) {
        const float *cn = pass ? c : NULL;
        oracle_prune24_mask(w, cn, N, K, keep);
        oracle_prune24_compress_tensor(w, cn, N, K, vals, meta, s2);
        for (int64_t i = 1; i < (N / 128) * (K / 128); i++)
            if (s2[i] != s2[0]) bad |= fail("one tensor scale");
        oracle_prune24_compress(w, cn, N, K, vals, meta, s2);
        oracle_decompress24(vals, meta, N, K, dq);
        for (int64_t i = 0; i < N * K; i += 4) {
            int kept = keep[i] + keep[i + 1] + keep[i + 2] + keep[i + 3];
            if (kept != 2) bad |= fail("two kept per group");
        }
        for (int64_t i = 0; i < N * K; i++)
            if (!keep[i] && dq[i] != 0) bad |= fail("pruned positions decompress to code 0");
    }
    oracle_quant_act(x, M, K, xq, xs);
    oracle_quant_wblock(w, N, K, wq, ws);
    /* the GEMM on finite codes only (the random bf16 data may saturate, never NaN) */
    oracle_gemm(xq, xs, wq, ws, M, N, K, y);
    int64_t rows[3] = {M - 1, 0, M / 2};
    oracle_gemm_rows(xq, xs, wq, ws, M, N, K, rows, 3, yr);
    for (int r = 0; r < 3; r++)
        for (int64_t n = 0; n < N; n++) {
            const double a = yr[r * N + n], b = y[rows[r] * N + n];
            if (!(a == b || (isnan(a) && isnan(b)))) bad |= fail("gemm_rows equals gemm");
        }
    free(x); free(w); free(c); free(xq); free(wq); free(keep); free(xs); free(ws); free(xe); free(we);
    free(vals); free(meta); free(dq); free(s2); free(y); free(yr);
    return bad;
}

int main(void) {
    int bad = 0;
    for (int c = 0; c < 256; c++) {
        const double v = oracle_e4m3_decode((uint8_t)c);
        if (!isnan(v) && oracle_e4m3_encode(v) != (c == 0x80 ? 0x80 : c)) bad |= fail("encode(decode(c)) == c");
    }
    if (oracle_e4m3_encode(INFINITY) != 0x7E || oracle_e4m3_encode(-1e30) != 0xFE) bad |= fail("saturation");
    bad |= run_shape(3, 128, 128);
    bad |= run_shape(5, 256, 384);
    bad |= run_shape(1, 384, 256);
    if (oracle_num_threads() < 1) bad |= fail("threads");
    if (!bad) printf("oracle sanitizer driver: ok\n");
    return bad;
}
