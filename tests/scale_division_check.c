/* Enumeration check of the quantizer's reciprocal division.
 *
 * The dynamic per-tensor quantizer divides every element by one scale
 * s = amax / 448 (IEEE division) and encodes the quotient to E4M3. The GPU
 * kernels compute the quotient as q' = fma(fma(-q, s, x), y, q) with
 * q = x * y, y = 1 / s, and the sign taken from x, for 2^-90 <= s <= 2^90.
 * This program checks, for every finite nonzero 16-bit amax (bf16 or f16)
 * whose scale lies in that range and every 16-bit x with |x| <= amax, that
 * q' is the IEEE quotient x / s bit for bit wherever |x / s| >= 2^-10 (E4M3
 * rounding sends every magnitude below 2^-10 to zero); where |x / s| < 2^-10
 * (tiny x, whose residual may underflow) the check is that |q'| < 2^-10 too,
 * with the sign of x, so both encode to the same signed zero. Exit status 0
 * iff no pair fails. Usage: scale_division_check <bf16|f16>
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float from_bf16(uint32_t b) { return u2f(b << 16); }

static float from_f16(uint32_t h) {
    uint32_t s = (h >> 15) & 1u, e = (h >> 10) & 31u, m = h & 1023u;
    float v;
    if (e == 0) v = ldexpf((float)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexpf((float)(m | 1024u), (int)e - 25);
    return s ? -v : v;
}

int main(int argc, char** argv) {
    const int f16 = argc > 1 && strcmp(argv[1], "f16") == 0;
    long long tested = 0, bad = 0, scales = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : tested, bad, scales)
    for (int ab = 1; ab < 0x8000; ++ab) {
        const float amax = f16 ? from_f16((uint32_t)ab) : from_bf16((uint32_t)ab);
        if (!isfinite(amax)) continue;
        const float s = amax / 448.0f;
        if (!(s >= 0x1p-90f && s <= 0x1p90f)) continue;
        ++scales;
        const float y = 1.0f / s;
        for (uint32_t xb = 0; xb < 0x10000u; ++xb) {
            const float x = f16 ? from_f16(xb) : from_bf16(xb);
            if (isnan(x) || fabsf(x) > amax) continue;
            const float q = x * y;
            const float r = fmaf(-q, s, x);
            const float q2 = copysignf(fmaf(r, y, q), x);
            const float exact = x / s;
            ++tested;
            int ok;
            if (fabsf(exact) >= 0x1p-10f)
                ok = f2u(q2) == f2u(exact);
            else
                ok = fabsf(q2) < 0x1p-10f && signbit(q2) == signbit(x) && signbit(exact) == signbit(x);
            if (!ok) {
                ++bad;
                if (bad < 5)
#pragma omp critical
                    printf("differs: amax=%a x=%a s=%a x/s=%a q'=%a\n", amax, x, s, exact, q2);
            }
        }
    }
    printf("%s: %lld scales, %lld (amax, x) pairs, %lld differ\n", f16 ? "f16" : "bf16", scales, tested, bad);
    return bad != 0;
}
