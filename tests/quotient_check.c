/*
 * Exhaustive check of the quantizers' fast quotient, in IEEE single precision.
 *
 * The GPU quantizers encode x / s, with s = fl(amax / 448) and amax the
 * largest |x| of a group (a bf16 value), as
 *     rs = fl(1 / s),  q0 = fl(x * rs),  q = fma(-fma(q0, s, -x), rs, q0)
 * and claim that the e4m3 code of q equals that of the correctly rounded
 * quotient fl(x / s) whenever amax >= 2^-90.  check_range enumerates every
 * bf16 amax in [a_lo, a_hi) and every bf16 x with |x| <= amax, of both signs
 * (the signs of zero results are not symmetric), and counts the pairs whose
 * codes differ.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (plus -mfma where
 * the CPU has it; fmaf is exact either way).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float from_bits(uint32_t u) {
    float x;
    memcpy(&x, &u, 4);
    return x;
}

/* OCP E4M3FN code of a finite fp32 value: round to nearest even on the e4m3
 * grid (subnormal spacing 2^-9 below 2^-6, 3 mantissa bits above), saturating
 * at 448.  Written from the format's definition, independently of the
 * library and of the oracle (the test compares it with the oracle). */
int e4m3_code(float v) {
    const int sign = signbit(v) ? 0x80 : 0;
    const double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7E;
    int e;
    double spacing;
    if (a < 0x1p-6) {
        spacing = 0x1p-9;
    } else {
        frexp(a, &e); /* a = f * 2^e, 0.5 <= f < 1 */
        spacing = ldexp(1.0, e - 4);
    }
    const double n = a / spacing; /* exact: spacing is a power of two */
    const double fl = floor(n), rem = n - fl;
    const double r = rem > 0.5 ? fl + 1 : rem < 0.5 ? fl : (fmod(fl, 2.0) == 0.0 ? fl : fl + 1);
    const double val = r * spacing;
    if (val >= 448.0) return sign | 0x7E;
    if (val < 0x1p-6) return sign | (int)(val / 0x1p-9);
    frexp(val, &e);
    const int biased = e - 1 + 7, mant = (int)(val / ldexp(1.0, e - 1) * 8.0) - 8;
    return sign | (biased << 3) | mant;
}

/* Pairs (amax, x) with amax in [a_lo, a_hi) (bf16 bit patterns of positive
 * finite values) whose fast and exact codes differ; *largest gets the
 * largest such amax pattern (0 if none). */
int64_t check_range(uint32_t a_lo, uint32_t a_hi, uint32_t *largest) {
    int64_t bad = 0;
    uint32_t top = 0;
#pragma omp parallel for reduction(+ : bad) reduction(max : top) schedule(dynamic, 64)
    for (uint32_t a = a_lo; a < a_hi; a++) {
        const float amax = from_bits(a << 16);
        const float s = amax / 448.0f;
        const float rs = 1.0f / s;
        int64_t b = 0;
        for (uint32_t xb = 0; xb <= a; xb++) {
            for (uint32_t sign = 0; sign <= 0x8000u; sign += 0x8000u) {
                const float x = from_bits((xb | sign) << 16);
                const float q0 = x * rs;
                /* volatile: the remainder must be rounded before it is
                 * negated (folding the negation into this fma would turn
                 * -(+0) into +0 for x = -0) */
                volatile float r = fmaf(q0, s, -x);
                const float q = fmaf(-r, rs, q0);
                const float exact = x / s;
                if (e4m3_code(q) != e4m3_code(exact)) b++;
            }
        }
        if (b) {
            bad += b;
            if (a > top) top = a;
        }
    }
    *largest = top;
    return bad;
}
