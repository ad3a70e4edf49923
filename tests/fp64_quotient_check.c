/* Check of the fused RMSNorm quantizers' fp32 division.
 *
 * The kernels divide a finite fp32 y by a finite scale s > 0 as
 *   inv = 1/s rounded to fp64,  q = fp32(fp64(y * inv)).
 * The claim: q is the IEEE quotient y / s bit for bit whenever y / s is in
 * the fp32 normal range; below it both quotients are below 2^-126 in
 * magnitude with the sign of y (every quantization code is then zero).
 * The argument: fp64(y * inv) is within 2^-52 (relative) of y / s; an exact
 * quotient is never an fp32 rounding boundary (a midpoint needs a 25-bit odd
 * significand, and y = m * s would give y an odd part that wide), and a
 * non-boundary quotient lies at least 2^-49 (relative) from every boundary.
 * This program tests the claim on random pairs over the whole fp32 range,
 * on the quantizers' own range (s = amax/448 or amax/127, |y| <= amax), on
 * pairs whose quotient lies next to a boundary (y = fp32(m * s) for a
 * midpoint m and its neighbours), and on subnormal y; it also reports the
 * smallest distance, in units of 2^-52 relative, between a sampled quotient
 * and its nearest boundary.  Exit status 0 iff nothing fails.
 * Usage: fp64_quotient_check <pairs>
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {  /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static long long tested, bad;
static double min_gap = 1e300;  /* in units of 2^-52 of |y/s| */

static void check(float y, float s) {
    if (!isfinite(y) || !isfinite(s) || !(s > 0.0f)) return;
    const float ref = y / s;  /* IEEE fp32 division */
    if (!isfinite(ref)) return;
    const double inv = 1.0 / (double)s;
    const float q = (float)((double)y * inv);
    ++tested;
    if (fabsf(ref) >= 0x1p-126f) {
        if (f2u(q) != f2u(ref)) {
            if (bad < 10) printf("differ: y=%a s=%a ieee=%a fast=%a\n", y, s, ref, q);
            ++bad;
        }
        /* distance of the exact quotient from the nearest boundary, from
         * the exact residual y - b*s of each neighbouring boundary b (b*s
         * has at most 49 bits, so fma gives it exactly) */
        const float a = fabsf(ref);
        const double lo = ((double)a + (double)u2f(f2u(a) - 1u)) / 2.0;  /* boundaries next to a */
        const double hi = ((double)a + (double)u2f(f2u(a) + 1u)) / 2.0;
        const double ay = fabs((double)y);
        const double g = fmin(fabs(fma(-lo, (double)s, ay)), fabs(fma(-hi, (double)s, ay))) /
                         (double)s / (double)a / 0x1p-52;
        if (g < min_gap) min_gap = g;
    } else if (!(fabsf(q) <= 0x1p-126f) || signbit(q) != signbit(y)) {
        if (bad < 10) printf("tiny differ: y=%a s=%a ieee=%a fast=%a\n", y, s, ref, q);
        ++bad;
    }
}

static float rand_float(int lo_exp, int hi_exp) {
    const int e = lo_exp + (int)(next_u64() % (uint64_t)(hi_exp - lo_exp + 1));
    const uint32_t m = (uint32_t)next_u64() & 0x7FFFFFu;
    const uint32_t sgn = (uint32_t)(next_u64() & 1u) << 31;
    return u2f(sgn | ((uint32_t)(e + 127) << 23) | m);
}

int main(int argc, char** argv) {
    const long long pairs = argc > 1 ? atoll(argv[1]) : 10000000;
    for (long long i = 0; i < pairs; ++i)  /* whole range */
        check(rand_float(-126, 100), fabsf(rand_float(-126, 100)));
    for (long long i = 0; i < pairs; ++i) {  /* the quantizers' range */
        const float amax = fabsf(rand_float(-60, 60));
        const float s = (next_u64() & 1) ? amax / 448.0f : amax / 127.0f;
        const float y = u2f(f2u(amax) - (uint32_t)(next_u64() % 0x3000000u)) * ((next_u64() & 1) ? -1.f : 1.f);
        check(y, s);
        check(amax, s);
    }
    for (long long i = 0; i < pairs; ++i) {  /* quotients next to a boundary */
        const float s = fabsf(rand_float(-60, 60));
        const uint32_t mm = ((((uint32_t)next_u64() & 0x7FFFFFu) | 0x800000u) << 1) | 1u;
        const double m = ldexp((double)mm, -24 + (int)(next_u64() % 60u) - 30);
        const float y = (float)(m * (double)s);
        check(y, s);
        check(u2f(f2u(y) + 1u), s);
        check(u2f(f2u(y) - 1u), s);
    }
    for (long long i = 0; i < pairs / 10; ++i)  /* subnormal y */
        check(u2f((uint32_t)next_u64() & 0x807FFFFFu), fabsf(rand_float(-126, 20)));
    printf("%lld pairs, %lld differ, smallest quotient-to-boundary gap %.3g x 2^-52 (needs > 1)\n",
           tested, bad, min_gap);
    return bad == 0 && min_gap > 1.0 ? 0 : 1;
}
