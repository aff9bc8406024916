/*
 * Host replay of the requantizer kernel's division step (tests only).
 *
 * The kernel needs fp32(a / b) for a dequantized value a (any fp32) and a
 * column-tile scale b.  For 2^-60 <= b <= 2^60 it computes, with one IEEE
 * division per column and five operations per element:
 *   rh = fp32(1 / b)                 (IEEE division)
 *   rl = fp32(fma(-rh, b, 1) * rh)   (the residual 1 - b*rh is exact, so
 *                                     rh + rl = 1/b within 2^-47 relative)
 *   y  = fma(a, rh, fp32(a * rl))    (within 0.5 ulp + 2^-46 relative of a/b:
 *                                     a faithful quotient)
 *   e  = fma(-y, b, a)               (exact residual of a faithful quotient)
 *   z  = fma(e, rh, y)               (Markstein's correction: with y faithful
 *                                     and rh the rounded reciprocal it gives
 *                                     the correctly rounded quotient)
 *   q  = copysign(z, a)
 * The argument needs no underflow, which the scale range guarantees whenever
 * |a / b| >= 2^-12; below that only the zero code of the right sign matters.
 *
 * Without underflow the steps commute with scaling a or b by powers of two,
 * so the result depends only on the two significands.  This program checks
 *   1. every numerator significand (2^23 values) against 256 divisor
 *      significands (special ones and pseudo-random ones), for one binade of
 *      the quotient on each side of 1: z must equal a / b bit for bit;
 *   2. 2^27 pseudo-random pairs over the whole kernel domain: b anywhere in
 *      [2^-60, 2^60], |a| from the smallest subnormal to 449 b, both signs:
 *      q must equal a / b bit for bit when |a / b| >= 2^-12, and otherwise
 *      both must lie below 2^-10 in magnitude with the sign of a (the same
 *      e4m3 code).
 * Prints the number of checked pairs and of violations.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float fu(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t uf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static uint64_t mix(uint64_t x)
{
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

static float fast_quot(float a, float b, float rh, float rl)
{
    float y = fmaf(a, rh, a * rl);
    float e = fmaf(-y, b, a);
    float z = fmaf(e, rh, y);
    return copysignf(z, a);
}

static int ok(float a, float b, float q)
{
    float ref = a / b;
    if (fabsf(ref) >= 0x1p-12f)
        return uf(q) == uf(ref);
    return fabsf(q) < 0x1p-10f && signbit(q) == signbit(a);
}

int main(void)
{
    long long pairs = 0, bad = 0;
    enum { NDIV = 256 };
    uint32_t divsig[NDIV];
    int i, n = 0;
    /* special divisor significands: 1, 1 + ulp, 2 - ulp, few-bit patterns, 1/448-like */
    const uint32_t special[] = {0x000000, 0x000001, 0x7FFFFF, 0x400000, 0x7FFFFE, 0x000002,
                                0x600000, 0x200000, 0x555555, 0x2AAAAA, 0x124925, 0x492492,
                                0x6DB6DB, 0x36DB6E};
    for (i = 0; i < (int)(sizeof special / sizeof special[0]); ++i)
        divsig[n++] = special[i];
    /* significands of fp32(amax / 448) for amax = 448 * (1 + k/8) (e4m3-like maxima) */
    for (i = 0; i < 8; ++i)
        divsig[n++] = uf((448.0f * (1.0f + i / 8.0f)) / 448.0f) & 0x7FFFFF;
    for (i = 0; i < 64; ++i)
        divsig[n++] = uf(fu(0x43000000u | (uint32_t)(mix(i) & 0x7FFFFF)) / 448.0f) & 0x7FFFFF;
    while (n < NDIV) {
        divsig[n] = (uint32_t)(mix(1000 + n) & 0x7FFFFF);
        ++n;
    }

    /* 1. exhaustive numerator significands */
#pragma omp parallel for reduction(+:pairs, bad) schedule(dynamic, 1)
    for (i = 0; i < NDIV; ++i) {
        float b = fu(0x3F800000u | divsig[i]);       /* [1, 2) */
        float rh = 1.0f / b;
        float rl = fmaf(-rh, b, 1.0f) * rh;
        uint32_t m;
        for (m = 0; m < (1u << 23); ++m) {
            float a1 = fu(0x3F800000u | m);          /* [1, 2): quotient in (0.5, 2) */
            float a2 = fu(0x43000000u | m);          /* [128, 256) */
            pairs += 2;
            if (!ok(a1, b, fast_quot(a1, b, rh, rl))) bad++;
            if (!ok(a2, b, fast_quot(a2, b, rh, rl))) bad++;
        }
    }

    /* 2. random pairs over the kernel's domain */
#pragma omp parallel for reduction(+:pairs, bad) schedule(static)
    for (i = 0; i < 1024; ++i) {
        int j;
        for (j = 0; j < (1 << 17); ++j) {
            uint64_t h = mix(((uint64_t)i << 32) | (uint64_t)j);
            int eb = (int)(h % 121) - 60;                          /* b in [2^-60, 2^61) */
            float b = ldexpf(fu(0x3F800000u | (uint32_t)((h >> 8) & 0x7FFFFF)), eb);
            uint64_t h2 = mix(h);
            /* |a| = 449 b * 2^-t, t uniform in [0, 200): covers the subnormals */
            double t = (double)(h2 % 200000) / 1000.0;
            float a, rh, rl;
            if (b > 0x1p60f)
                b = 0x1p60f;
            a = (float)(449.0 * (double)b * pow(2.0, -t));
            if (h2 & 1)
                a = -a;
            rh = 1.0f / b;
            rl = fmaf(-rh, b, 1.0f) * rh;
            pairs++;
            if (!ok(a, b, fast_quot(a, b, rh, rl))) bad++;
        }
    }
    printf("%lld %lld\n", pairs, bad);
    return 0;
}
