/* Exhaustive check of the block-scale quotient the NVFP4 encoders use on the
 * GPU: for every finite fp32 a >= 2^-125, q0 = RN(a * RN(1/6)),
 * r = fma(-q0, 6, a), q1 = fma(r, RN(1/6), q0) equals the IEEE quotient
 * RN(a / 6); and below 2^-125 both quotients times any S <= 2^100 stay under
 * 2^-10 (half the smallest E4M3 step), so the scale byte is 0 either way.
 * Prints "mismatches N small_bad M" and exits 0 when both are 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void) {
    const float y = 1.0f / 6.0f;
    const float smax = ldexpf(1.0f, 100), half_step = ldexpf(1.0f, -10);
    long long bad = 0, small_bad = 0;
#pragma omp parallel for reduction(+ : bad, small_bad) schedule(static, 1 << 20)
    for (long long i = 0; i < 0x7F800000LL; ++i) {
        const float a = from_bits((uint32_t)i);
        const float ref = a / 6.0f;
        const float q0 = a * y;
        const float r = fmaf(-q0, 6.0f, a);
        const float q1 = fmaf(r, y, q0);
        if (i >= 0x01000000LL) {
            if (to_bits(q1) != to_bits(ref)) ++bad;
        } else if (!(q1 * smax < half_step && ref * smax < half_step)) {
            ++small_bad;
        }
    }
    printf("mismatches %lld small_bad %lld\n", bad, small_bad);
    return (bad || small_bad) ? 1 : 0;
}
