/*
 * Host replay of the quantizer kernels' division step (tests only).
 *
 * The kernels compute fp32(x / s) for a tile with scale s >= 2^-73 as
 *   r = fp32(1 / s)            (IEEE division, once per tile)
 *   y = fp32(x * r)
 *   e = fma(-y, s, x)          (exact residual)
 *   z = fma(e, r, y)           (one correction step)
 *   q = copysign(z, x)
 * and divide directly for smaller scales.  This program walks every pair of
 * bf16 values (x, amax) with |x| <= amax and s = fp32(amax / 448) >= 2^-73,
 * both signs of x, and checks that q equals the IEEE quotient x / s bit for
 * bit whenever |x / s| >= 2^-12, and otherwise that both are below 2^-10 in
 * magnitude with the same sign -- so that both map to the same e4m3 code
 * (the zero code of that sign).  Prints the number of violations.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf(uint32_t h) { uint32_t u = h << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t fb(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void)
{
    long long bad = 0, pairs = 0;
    int ab;
#pragma omp parallel for reduction(+:bad, pairs) schedule(dynamic, 64)
    for (ab = 1; ab < 0x7F80; ++ab) {
        float amax = bf((uint32_t)ab);
        float s = amax / 448.0f;
        float r;
        int xb, sg;
        if (!(s >= 0x1p-73f))
            continue;
        r = 1.0f / s;
        for (xb = 0; xb <= ab; ++xb)
            for (sg = 0; sg < 2; ++sg) {
                float x = bf((uint32_t)xb | (sg ? 0x8000u : 0u));
                float ref = x / s;
                float y = x * r;
                float e = fmaf(-y, s, x);
                float q = copysignf(fmaf(e, r, y), x);
                pairs++;
                if (fabsf(ref) >= 0x1p-12f) {
                    if (fb(q) != fb(ref)) bad++;
                } else if (!(fabsf(q) < 0x1p-10f && signbit(q) == signbit(ref))) {
                    bad++;
                }
            }
    }
    printf("%lld %lld\n", pairs, bad);
    return 0;
}
