/*
 * CPU oracle for the FP8 quantized linear layer (dense block-scaled and 2:4
 * sparse).  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the CPU
 * baseline leg of the benchmark may call it; the library never does.  It shares
 * no code, header, table or helper with the HIP path.
 *
 * Plain, slow and written to be checked by eye against the definitions:
 *
 *  - "FP8 a granularite fine" (Hugging Face transformers docs), intro bullets:
 *    weights are quantized to 8 bits per 2-D block of 128x128, activations to
 *    8 bits per token in groups of 128 input channels; section "Chemin rapide
 *    de DeepGEMM": the activation scheme is dynamic (scale computed from the
 *    live group).
 *  - "Deployer la parcimonie 2:4 avec FP8 sur Hopper" (mtechresearch), pipeline
 *    step 2 (groups of 4 contiguous values along K), step 4 (magnitude or
 *    activation-aware scores, drop the 2 least important of each 4), step 6
 *    (recalibrate the FP8 scales after pruning), step 7 (export pruned weights
 *    with their 2:4 masks); "Exemples pratiques" example 1 (top-2 of |w| per
 *    group of 4 along dim 1 of nn.Linear.weight).
 *  - "Combiner elagage et quantification..." (eva-circle), "La cle : la
 *    sparsite structuree 2:4": keep the two largest of every four.
 *
 * The pages do not fix the FP8 bit format, the rounding, the scale formula or
 * the tie rule; this oracle uses:
 *  - OCP FP8 E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 *    infinities, NaN = S.1111.111, largest finite 448;
 *  - encode = round to nearest, ties to the even code, saturating at +-448;
 *  - scale s = amax / 448 as an IEEE fp32 division; codes = enc(fp32(x / s))
 *    where x / s is also an IEEE fp32 division (the scale is an fp32 number);
 *  - amax == 0 gives s == 0 and codes that are signed zeros;
 *  - 2:4 ties keep the lower index.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -fno-fast-math -ffp-contract=off -shared -fPIC
 * (no flush-to-zero: the fp32 scale may be subnormal).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define G 128 /* group / block edge */

/* ---------------------------------------------------------------- bf16 ---- */

/* bf16 bits -> fp32: the bf16 pattern is the top half of the fp32 pattern. */
static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ---------------------------------------------------------------- e4m3 ---- */

/* Decode one E4M3FN code by the closed form of the format. */
double oracle_e4m3_decode(uint8_t c) {
    int S = c >> 7, E = (c >> 3) & 15, F = c & 7;
    double v;
    if (E == 15 && F == 7) return NAN;
    if (E == 0)
        v = F * ldexp(1.0, -9); /* subnormal: F/8 * 2^(1-7) */
    else
        v = (1.0 + F / 8.0) * ldexp(1.0, E - 7);
    return S ? -v : v;
}

/* The 127 non-negative finite values in increasing order (codes 0x00..0x7E). */
static double e4m3_pos[127];

__attribute__((constructor)) static void init_e4m3_table(void) {
    for (int c = 0; c < 127; c++) e4m3_pos[c] = oracle_e4m3_decode((uint8_t)c);
}

/*
 * Encode a real value (given as a double) to E4M3FN, round to nearest with
 * ties to the even code, saturating.  A bisection over the 127 non-negative
 * finite values finds the neighbours lo <= |v| <= hi; |v| is then compared
 * with their midpoint (midpoints have 5 significant bits, so they and the
 * comparison are exact in double).
 */
uint8_t oracle_e4m3_encode(double v) {
    uint8_t S = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (isnan(v)) return S | 0x7F;
    if (a >= 448.0) return S | 0x7E;
    int lo = 0, hi = 126; /* invariant: e4m3_pos[lo] <= a < e4m3_pos[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (e4m3_pos[mid] <= a) lo = mid; else hi = mid;
    }
    double m = (e4m3_pos[lo] + e4m3_pos[hi]) / 2.0;
    if (a < m) return S | (uint8_t)lo;
    if (a > m) return S | (uint8_t)hi;
    return S | (uint8_t)((lo % 2 == 0) ? lo : hi); /* tie: even code */
}

/* The value of one input divided by its scale, then encoded. */
static uint8_t quantize_one(float x, float s) {
    if (s == 0.0f) return signbit(x) ? 0x80 : 0x00; /* amax == 0 */
    float r = x / s;                                 /* IEEE fp32 division */
    return oracle_e4m3_encode((double)r);
}

/* ------------------------------------------------- activation quantization */

/*
 * Per token m and group kb of 128 channels: amax = max |x|, s = amax/448 (fp32),
 * q = enc(x / s).  X [M,K] bf16 bits, row-major; Q [M,K]; S [M,K/128].
 */
void oracle_quant_act(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s) {
    int64_t KB = K / G;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t kb = 0; kb < KB; kb++) {
            float amax = 0.0f;
            for (int64_t k = kb * G; k < (kb + 1) * G; k++) {
                float a = fabsf(bf16_to_f32(x[m * K + k]));
                if (a > amax) amax = a;
            }
            float sc = amax / 448.0f;
            s[m * KB + kb] = sc;
            for (int64_t k = kb * G; k < (kb + 1) * G; k++)
                q[m * K + k] = quantize_one(bf16_to_f32(x[m * K + k]), sc);
        }
    }
}

/* ---------------------------------------------- weight block quantization */

/*
 * Per 128x128 block (nb,kb) of W [N,K]: amax over the block, s = amax/448 (fp32),
 * q = enc(w / s).  S is [N/128, K/128] row-major.
 */
void oracle_quant_wblock(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s) {
    int64_t NB = N / G, KB = K / G;
#pragma omp parallel for schedule(static)
    for (int64_t nb = 0; nb < NB; nb++) {
        for (int64_t kb = 0; kb < KB; kb++) {
            float amax = 0.0f;
            for (int64_t n = nb * G; n < (nb + 1) * G; n++)
                for (int64_t k = kb * G; k < (kb + 1) * G; k++) {
                    float a = fabsf(bf16_to_f32(w[n * K + k]));
                    if (a > amax) amax = a;
                }
            float sc = amax / 448.0f;
            s[nb * KB + kb] = sc;
            for (int64_t n = nb * G; n < (nb + 1) * G; n++)
                for (int64_t k = kb * G; k < (kb + 1) * G; k++)
                    q[n * K + k] = quantize_one(bf16_to_f32(w[n * K + k]), sc);
        }
    }
}

/* ------------------------------------------------------------- 2:4 pruning */

/*
 * Mask of W [N,K]: for row n and group g of 4 contiguous values along K,
 * score_j = |w[n,4g+j]| * c[4g+j] (c == NULL: c = 1), formed in fp64, where the
 * product of a bf16 and an fp32 is exact.  The indices are sorted by score,
 * largest first, with a stable insertion sort (equal scores keep index order),
 * and the first two are kept.  keep [N,K] receives 1 for kept, 0 for dropped.
 */
void oracle_prune24_mask(const uint16_t *w, const float *c, int64_t N, int64_t K, uint8_t *keep) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t g = 0; g < K / 4; g++) {
            double sc[4];
            int idx[4] = {0, 1, 2, 3};
            for (int j = 0; j < 4; j++) {
                int64_t k = 4 * g + j;
                double mag = fabs((double)bf16_to_f32(w[n * K + k]));
                sc[j] = mag * (c ? (double)c[k] : 1.0);
            }
            for (int i = 1; i < 4; i++)
                for (int j = i; j > 0 && sc[idx[j - 1]] < sc[idx[j]]; j--) {
                    int t = idx[j - 1];
                    idx[j - 1] = idx[j];
                    idx[j] = t;
                }
            for (int j = 0; j < 4; j++) keep[n * K + 4 * g + j] = 0;
            keep[n * K + 4 * g + idx[0]] = 1;
            keep[n * K + 4 * g + idx[1]] = 1;
        }
    }
}

/*
 * Prune, re-derive the block scales over the kept values, quantize the kept
 * values and compress.  For group g of row n with kept indices i0 < i1:
 *   vals[n, 2g] = code of w[n,4g+i0],  vals[n, 2g+1] = code of w[n,4g+i1],
 *   nibble = i0 | (i1 << 2), stored in meta[n, g/2] at bits 4*(g%2) .. +3.
 * vals [N,K/2], meta [N,K/8], s [N/128,K/128].
 */
void oracle_prune24_compress(const uint16_t *w, const float *c, int64_t N, int64_t K,
                             uint8_t *vals, uint8_t *meta, float *s) {
    int64_t NB = N / G, KB = K / G;
    uint8_t *keep = (uint8_t *)malloc((size_t)(N * K));
    oracle_prune24_mask(w, c, N, K, keep);
    /* block scales over the pruned matrix (dropped entries are zero) */
#pragma omp parallel for schedule(static)
    for (int64_t nb = 0; nb < NB; nb++)
        for (int64_t kb = 0; kb < KB; kb++) {
            float amax = 0.0f;
            for (int64_t n = nb * G; n < (nb + 1) * G; n++)
                for (int64_t k = kb * G; k < (kb + 1) * G; k++) {
                    float a = keep[n * K + k] ? fabsf(bf16_to_f32(w[n * K + k])) : 0.0f;
                    if (a > amax) amax = a;
                }
            s[nb * KB + kb] = amax / 448.0f;
        }
    memset(meta, 0, (size_t)(N * K / 8));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t g = 0; g < K / 4; g++) {
            float sc = s[(n / G) * KB + (4 * g) / G];
            int kept[2], nk = 0;
            for (int j = 0; j < 4; j++)
                if (keep[n * K + 4 * g + j]) kept[nk++] = j;
            vals[n * (K / 2) + 2 * g] = quantize_one(bf16_to_f32(w[n * K + 4 * g + kept[0]]), sc);
            vals[n * (K / 2) + 2 * g + 1] = quantize_one(bf16_to_f32(w[n * K + 4 * g + kept[1]]), sc);
            uint8_t nib = (uint8_t)(kept[0] | (kept[1] << 2));
            meta[n * (K / 8) + g / 2] |= (uint8_t)(nib << (4 * (g % 2)));
        }
    free(keep);
}

/*
 * The same prune and compression with one scale for the whole tensor
 * ("Deployer la parcimonie 2:4 avec FP8 sur Hopper": pipeline step 3, FP8 with
 * a per-tensor scale; step 6, the scale re-derived after pruning): amax over
 * every kept value of W, s = amax / 448 (fp32), kept codes enc(fp32(w / s)),
 * s written to every entry of the [N/128, K/128] scale array.
 */
void oracle_prune24_compress_tensor(const uint16_t *w, const float *c, int64_t N, int64_t K,
                                    uint8_t *vals, uint8_t *meta, float *s) {
    int64_t NB = N / G, KB = K / G;
    uint8_t *keep = (uint8_t *)malloc((size_t)(N * K));
    oracle_prune24_mask(w, c, N, K, keep);
    float amax = 0.0f;
    for (int64_t i = 0; i < N * K; i++) {
        float a = keep[i] ? fabsf(bf16_to_f32(w[i])) : 0.0f;
        if (a > amax) amax = a;
    }
    float sc = amax / 448.0f;
    for (int64_t i = 0; i < NB * KB; i++) s[i] = sc;
    memset(meta, 0, (size_t)(N * K / 8));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t g = 0; g < K / 4; g++) {
            int kept[2], nk = 0;
            for (int j = 0; j < 4; j++)
                if (keep[n * K + 4 * g + j]) kept[nk++] = j;
            vals[n * (K / 2) + 2 * g] = quantize_one(bf16_to_f32(w[n * K + 4 * g + kept[0]]), sc);
            vals[n * (K / 2) + 2 * g + 1] = quantize_one(bf16_to_f32(w[n * K + 4 * g + kept[1]]), sc);
            uint8_t nib = (uint8_t)(kept[0] | (kept[1] << 2));
            meta[n * (K / 8) + g / 2] |= (uint8_t)(nib << (4 * (g % 2)));
        }
    free(keep);
}

/* Inverse of the packing: dense codes [N,K] with 0x00 at the pruned places. */
void oracle_decompress24(const uint8_t *vals, const uint8_t *meta, int64_t N, int64_t K, uint8_t *q) {
    memset(q, 0, (size_t)(N * K));
    for (int64_t n = 0; n < N; n++)
        for (int64_t g = 0; g < K / 4; g++) {
            int nib = (meta[n * (K / 8) + g / 2] >> (4 * (g % 2))) & 15;
            int i0 = nib & 3, i1 = nib >> 2;
            q[n * K + 4 * g + i0] = vals[n * (K / 2) + 2 * g];
            q[n * K + 4 * g + i1] = vals[n * (K / 2) + 2 * g + 1];
        }
}

/* ------------------------------------------------------------------- GEMM */

/*
 * One output row: for each n and K block kb,
 *   P = sum_{k in kb} dec(qx[m,k]) * dec(qw[n,k])            (fp64, exact)
 *   y[m,n] = sum_kb (sx[m,kb] * sw[n/128,kb]) * P            (fp64)
 */
static void gemm_row(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                     int64_t m, int64_t N, int64_t K, const double *dec, double *yrow) {
    int64_t KB = K / G;
    for (int64_t n = 0; n < N; n++) {
        double acc = 0.0;
        for (int64_t kb = 0; kb < KB; kb++) {
            double P = 0.0;
            for (int64_t k = kb * G; k < (kb + 1) * G; k++)
                P += dec[xq[m * K + k]] * dec[wq[n * K + k]];
            acc += ((double)xs[m * KB + kb] * (double)ws[(n / G) * KB + kb]) * P;
        }
        yrow[n] = acc;
    }
}

/* Y [M,N] fp64 = block-dequantized X times W transposed; rows split over threads. */
void oracle_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                 int64_t M, int64_t N, int64_t K, double *y) {
    double dec[256];
    for (int c = 0; c < 256; c++) dec[c] = oracle_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; m++) gemm_row(xq, xs, wq, ws, m, N, K, dec, y + m * N);
}

/* The same for the listed rows only: y [R,N] holds rows[0..R) of Y. */
void oracle_gemm_rows(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                      int64_t M, int64_t N, int64_t K, const int64_t *rows, int64_t R, double *y) {
    double dec[256];
    (void)M;
    for (int c = 0; c < 256; c++) dec[c] = oracle_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; r++) gemm_row(xq, xs, wq, ws, rows[r], N, K, dec, y + r * N);
}

/* ------------------------------------- per-tensor and static act scales -- */

/*
 * Per-tensor activation scales ("Deployer la parcimonie 2:4 avec FP8 sur
 * Hopper", pipeline step 3 and "Bonnes pratiques": dynamic per-tensor FP8
 * scaling) and static scales ("FP8 a granularite fine", section "Chemin rapide
 * de DeepGEMM": a static activation scheme, the scale fixed beforehand).  Both
 * quantize every element with one scale s: q = enc(fp32(x / s)), saturating.
 * The dynamic per-tensor scale is s = fp32(amax / 448) over the whole tensor.
 * The scale is written to every entry of the [M, K/128] block-scale array, so
 * that the block-scaled GEMM takes these codes unchanged.
 */
void oracle_quant_act_static(const uint16_t *x, int64_t M, int64_t K, float s_in, uint8_t *q, float *s) {
    int64_t KB = K / G;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t k = 0; k < K; k++) q[m * K + k] = quantize_one(bf16_to_f32(x[m * K + k]), s_in);
        for (int64_t kb = 0; kb < KB; kb++) s[m * KB + kb] = s_in;
    }
}

void oracle_quant_act_tensor(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s) {
    float amax = 0.0f;
    for (int64_t i = 0; i < M * K; i++) {
        float a = fabsf(bf16_to_f32(x[i]));
        if (a > amax) amax = a;
    }
    oracle_quant_act_static(x, M, K, amax / 448.0f, q, s);
}

/* ------------------------------------------------------ UE8M0 scales ---- */

/*
 * Power-of-two scales stored as UE8M0 bytes ("FP8 a granularite fine", section
 * "Format d'echelle UE8M0": scales kept as float8_e8m0fnu).  A byte e stands
 * for 2^(e - 127).  The pages do not say how amax/448 becomes a power of two;
 * this oracle takes the smallest power of two that is not below amax/448, so
 * no value saturates: e is the smallest integer in [0, 254] with
 * 448 * 2^(e - 127) >= amax (e = 0 when amax is 0 or tiny).  Found here by a
 * plain upward search in double precision (448 * 2^(e - 127) is exact).
 */
static int ue8m0_exponent(double amax) {
    int e = 0;
    while (e < 254 && ldexp(448.0, e - 127) < amax) e++;
    return e;
}

/* code of x with scale 2^(e - 127): x * 2^(127 - e) is exact in double; one
 * rounding to e4m3 (never saturating, since |x| <= amax) */
static uint8_t quantize_one_ue8m0(float x, int e) {
    return oracle_e4m3_encode(ldexp((double)x, 127 - e));
}

void oracle_quant_act_ue8m0(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, uint8_t *e_out) {
    int64_t KB = K / G;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t kb = 0; kb < KB; kb++) {
            double amax = 0.0;
            for (int64_t k = kb * G; k < (kb + 1) * G; k++) {
                double a = fabs((double)bf16_to_f32(x[m * K + k]));
                if (a > amax) amax = a;
            }
            int e = ue8m0_exponent(amax);
            e_out[m * KB + kb] = (uint8_t)e;
            for (int64_t k = kb * G; k < (kb + 1) * G; k++)
                q[m * K + k] = quantize_one_ue8m0(bf16_to_f32(x[m * K + k]), e);
        }
    }
}

void oracle_quant_wblock_ue8m0(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, uint8_t *e_out) {
    int64_t NB = N / G, KB = K / G;
#pragma omp parallel for schedule(static)
    for (int64_t nb = 0; nb < NB; nb++) {
        for (int64_t kb = 0; kb < KB; kb++) {
            double amax = 0.0;
            for (int64_t n = nb * G; n < (nb + 1) * G; n++)
                for (int64_t k = kb * G; k < (kb + 1) * G; k++) {
                    double a = fabs((double)bf16_to_f32(w[n * K + k]));
                    if (a > amax) amax = a;
                }
            int e = ue8m0_exponent(amax);
            e_out[nb * KB + kb] = (uint8_t)e;
            for (int64_t n = nb * G; n < (nb + 1) * G; n++)
                for (int64_t k = kb * G; k < (kb + 1) * G; k++)
                    q[n * K + k] = quantize_one_ue8m0(bf16_to_f32(w[n * K + k]), e);
        }
    }
}

/* Threads OpenMP will use for the GEMM (reported with CPU timings). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
