/* Host check of the division identity the GPU quantisers use.
 *
 * For a per-tensor scale s in [2^-100, 2^100] with r = RN(1/s), the kernels
 * compute the quotient x / s of a bf16 value x as
 *     q0 = RN(x r),  q = RN(RN(q0 s - x) (-r) + q0)   (two fused multiply-adds)
 * and use q0 itself when it is infinite. The codes need q, clamped to +-448,
 * to equal the IEEE quotient RN(x / s) clamped the same way. This program
 * checks that:
 *   1. for every one of the 2^23 scale mantissas against every positive bf16
 *      mantissa (exponents where nothing under- or overflows: the identity
 *      then depends on the mantissas only), bit for bit;
 *   2. for every one of the 65536 bf16 bit patterns (zeros, subnormals,
 *      infinities and NaNs included) against a set of scales spanning the
 *      whole range, comparing the values that decide the e4m3 code: equal
 *      bits, both NaN, or both below 2^-12 in magnitude with the same sign
 *      (all of which round to a zero code of that sign).
 * Exit status 0 when no case differs. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float asf(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t asu(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float clamp448(float y) { return fminf(fmaxf(y, -448.f), 448.f); }

static float fast_quot(float x, float s, float r) {
    const float q0 = x * r;
    const float q1 = fmaf(fmaf(q0, s, -x), -r, q0);
    return isinf(q0) ? q0 : q1;
}

static uint32_t lcg = 12345u;
static uint32_t next_u32(void) { lcg = lcg * 1664525u + 1013904223u; return lcg; }

int main(void) {
    long bad = 0, n = 0;
    for (uint32_t sm = 0; sm < (1u << 23); ++sm) {
        const float s = asf((120u << 23) | sm);  /* [2^-7, 2^-6): static 6/448 lies here */
        const float r = 1.0f / s;
        for (uint32_t xm = 0; xm < 128; ++xm) {
            const float x = asf((127u << 23) | (xm << 16));
            const float a = clamp448(x / s), b = clamp448(fast_quot(x, s, r));
            ++n;
            if (asu(a) != asu(b)) {
                if (bad < 5) printf("mantissas: s=%a x=%a ieee=%a fast=%a\n", s, x, x / s, b);
                ++bad;
            }
        }
    }
    printf("mantissa pairs: %ld checked, %ld differ\n", n, bad);

    float scales[520];
    int ns = 0;
    scales[ns++] = 6.0f / 448.0f;
    scales[ns++] = 1e-12f / 448.0f;
    scales[ns++] = 0x1p-100f;
    scales[ns++] = 0x1p100f;
    scales[ns++] = 1.0f;
    scales[ns++] = 3.3895314e38f / 448.0f; /* largest bf16 over 448 */
    scales[ns++] = asf(0x3f7fffffu);
    scales[ns++] = asf(0x3f800001u);
    while (ns < 520) {
        /* exponents 2^-100 .. 2^100, any mantissa */
        const uint32_t e = 27u + next_u32() % 201u;
        scales[ns++] = asf((e << 23) | (next_u32() & 0x7fffffu));
    }
    long bad2 = 0, n2 = 0;
    for (int i = 0; i < ns; ++i) {
        const float s = scales[i], r = 1.0f / s;
        for (uint32_t h = 0; h < 65536u; ++h) {
            const float x = asf(h << 16);
            const float a = clamp448(x / s), b = clamp448(fast_quot(x, s, r));
            const int same = asu(a) == asu(b) || (isnan(a) && isnan(b)) ||
                             (fabsf(a) < 0x1p-12f && fabsf(b) < 0x1p-12f &&
                              signbit(a) == signbit(b));
            ++n2;
            if (!same) {
                if (bad2 < 5) printf("bf16 sweep: s=%a x=%a ieee=%a fast=%a\n", s, x, x / s, b);
                ++bad2;
            }
        }
    }
    printf("bf16 values x scales: %ld checked, %ld differ\n", n2, bad2);
    return (bad || bad2) ? 1 : 0;
}
