/*
 * CPU oracle for the quantized-linear hot path.  TEST INFRASTRUCTURE ONLY:
 * nothing in the product library calls, links or includes this file; only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * What it computes, and where the pages fix it:
 *  - OCP FP8 E4M3 ("FP8_E4M3 (OCP)" in the vLLM FP8 quantization-schema RFC,
 *    Scope list; torch.float8_e4m3fn in vLLM PR #4118, micro-benchmark
 *    legend and the follow-up summary).  The bit layout (bias 7, no infinity,
 *    S.1111.111 = NaN, max finite 448) is the OCP format the RFC names.
 *  - Dynamic per-tensor activation scaling (vLLM PR #4118, "Algorithm"):
 *    a fresh per-tensor scale every forward pass, scale = amax / 448, then a
 *    saturating round-to-nearest-even cast of x / scale.
 *  - Per-tensor weight scale computed after load (same section), and the
 *    per-output-channel weight scale vector of length N (optimum-quanto PR #241,
 *    the kernel's b_scales shape check: rank 2, (1, size_n)).
 *  - The FP8 GEMM Y = scale_a * scale_b * (Aq . Wq^T) with float accumulation
 *    (vLLM PR #4118, the torch._scaled_mm micro-benchmark description).
 *  - Weight-only fp8 (W8A16) linear with per-channel scales (optimum-quanto
 *    PR #241, "Marlin fp8").
 *  - W4A8 per-channel integer linear: int4 weights widened to int8 by a
 *    multiply by 16, int8 activations quantized per token, integer MMA,
 *    per-channel scale epilogue (QQQ issue #15, the answers on permutation,
 *    on "simply multiply 16" and on online activation quantization).
 *  - output_scale: an optional FP8 egress of a layer, quantized with a
 *    given output scale (vLLM FP8 quantization-schema RFC, the answer on
 *    output_scale).
 *  - RMSNorm followed by either activation quantizer (QQQ issue #15, the
 *    answer on online activation quantization fused into rmsnorm), with the
 *    precision reading stated at bqo_rmsnorm below.
 *  - Per-group W4A8, one scale per output channel and 128-k group (QQQ
 *    issue #15, the "qqq-g128" columns), with the reading stated at
 *    bqo_w4a8_group_linear below.
 *  - Per-group weight-only int4 (W4A16) with fp16 activations (QQQ issue
 *    #15, the "awq-g128" and "marlin-g128" columns), with the reading
 *    stated at bqo_w4a16_group_linear below.
 *
 * Readings where the pages are silent are ours and are listed in the design
 * notes: RNE, saturation to +-448, sign kept on zero/underflow, IEEE fp32
 * division x / scale, scale = 1 when amax = 0, a NaN in the tensor (row)
 * makes its E4M3 amax and scale NaN, int8 per-token scale = amax / 127 with
 * RNE and clamp to +-127 (NaN inputs outside its contract), low nibble =
 * even k for logical int4.
 *
 * Style: plain loops, no blocking, no reordering beyond the definitions.
 * OpenMP only splits independent output rows across host cores.
 * Build: gcc -O2 -fopenmp -fno-fast-math -ffp-contract=off -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BQO_F16 1
#define BQO_BF16 2
#define BQO_F32 3

/* Host threads the parallel loops below use. */
int bqo_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- E4M3 */

/* Decode one OCP E4M3 byte, bit by bit: sign, 4-bit exponent (bias 7),
 * 3-bit mantissa; exponent 0 is subnormal; S.1111.111 is NaN. */
double bqo_e4m3_decode(uint8_t c) {
    int s = (c >> 7) & 1;
    int e = (c >> 3) & 15;
    int m = c & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);              /* m/8 * 2^(1-7) */
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Encode a real value (given exactly as a double) to E4M3: the nearest
 * finite E4M3 value, ties to the code with an even mantissa, magnitudes at
 * or above 448 saturate to 448, the sign is always kept (so -0 and negative
 * underflow give 0x80).  The 127 non-negative finite codes 0x00..0x7E are
 * increasing in value, so the two neighbours are found by bisection. */
uint8_t bqo_e4m3_encode(double v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (isnan(v)) return sign | 0x7F;
    if (a >= 448.0) return sign | 0x7E;
    /* largest c in [0,126] with decode(c) <= a */
    int lo = 0, hi = 126; /* decode(lo) <= a < decode(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (bqo_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    double below = bqo_e4m3_decode((uint8_t)lo);
    double above = bqo_e4m3_decode((uint8_t)(lo + 1));
    double half = (below + above) / 2.0; /* exact: few significant bits */
    int c = lo;
    if (a > half) c = lo + 1;
    else if (a == half && (lo & 1)) c = lo + 1;   /* tie: even mantissa */
    return sign | (uint8_t)c;
}

/* ------------------------------------------------- 16-bit float inputs */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
float bqo_f16_to_f32(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double mag;
    if (e == 31) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)m, -24);
    else mag = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return (float)(s ? -mag : mag);
}

/* bfloat16 is the upper half of an IEEE binary32. */
float bqo_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

void bqo_decode_input(const void* x, int dtype, int64_t n, float* out) {
    const uint16_t* h = (const uint16_t*)x;
    for (int64_t i = 0; i < n; ++i) {
        if (dtype == BQO_F16) out[i] = bqo_f16_to_f32(h[i]);
        else if (dtype == BQO_BF16) out[i] = bqo_bf16_to_f32(h[i]);
        else out[i] = ((const float*)x)[i];
    }
}

/* ----------------------------------------------------- fp8 quantizers */

/* scale = amax / 448 in fp32 (one IEEE rounding); 1 when amax is 0. */
static float scale_from_amax(float amax, float qmax) {
    if (amax == 0.0f) return 1.0f;
    return amax / qmax;
}

/* max |x| over n values.  A NaN anywhere makes it NaN, as the maximum of a
 * torch tensor holding a NaN is NaN; the scale is then NaN and so is every
 * code of that tensor (row). */
static float amax_of(const float* x, int64_t n) {
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        if (isnan(x[i])) return NAN;
        if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
    }
    return amax;
}

/* Dynamic per-tensor quantization of n fp32 values. */
void bqo_quant_per_tensor(const float* x, int64_t n, uint8_t* q, float* scale_out) {
    float s = scale_from_amax(amax_of(x, n), 448.0f);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float r = x[i] / s;                     /* IEEE fp32 division */
        q[i] = bqo_e4m3_encode((double)r);
    }
    *scale_out = s;
}

/* Per-row (per output channel) quantization of a rows x cols matrix. */
void bqo_quant_per_row(const float* x, int64_t rows, int64_t cols, uint8_t* q,
                       float* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        float s = scale_from_amax(amax_of(xr, cols), 448.0f);
        for (int64_t k = 0; k < cols; ++k)
            q[r * cols + k] = bqo_e4m3_encode((double)(xr[k] / s));
        scales[r] = s;
    }
}

/* Quantize with caller-given scales: one scale per row (nscales == rows)
 * or one for the whole matrix (nscales == 1). */
void bqo_quant_with_scales(const float* x, int64_t rows, int64_t cols,
                           const float* scales, int64_t nscales, uint8_t* q) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float s = scales[nscales == 1 ? 0 : r];
        for (int64_t k = 0; k < cols; ++k)
            q[r * cols + k] = bqo_e4m3_encode((double)(x[r * cols + k] / s));
    }
}

/* --------------------------------------------------- int8 per-token */

/* Symmetric per-row int8: s[m] = amax_m / 127 (1 for a zero row),
 * q = clamp(round-half-even(x / s[m]), -127, 127). */
void bqo_int8_quant_per_token(const float* x, int64_t M, int64_t K, int8_t* q,
                              float* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const float* xr = x + m * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k)
            if (fabsf(xr[k]) > amax) amax = fabsf(xr[k]);
        float s = scale_from_amax(amax, 127.0f);
        for (int64_t k = 0; k < K; ++k) {
            float r = xr[k] / s;
            double t = nearbyint((double)r);   /* default mode: half to even */
            if (t > 127.0) t = 127.0;
            if (t < -127.0) t = -127.0;
            q[m * K + k] = (int8_t)t;
        }
        scales[m] = s;
    }
}

/* --------------------------------------------------------- int4 */

/* Logical int4 packing: two's-complement nibbles, two per byte along k,
 * the low nibble holding the even k.  Returns the int values -8..7. */
void bqo_unpack_int4(const uint8_t* packed, int64_t N, int64_t K, int8_t* w) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t b = packed[(n * K + k) / 2];
            int nib = (k % 2 == 0) ? (b & 15) : (b >> 4);
            w[n * K + k] = (int8_t)(nib >= 8 ? nib - 16 : nib);
        }
}

/* ---------------------------------------------------------- linears */

/* Exact fp8 dot products.  Every E4M3 value times 2^9 is an integer of
 * magnitude at most 229376, so sum_k (2^9 a)(2^9 w) is exact in int64 and
 * acc = that sum * 2^-18 exactly.  Rows listed in `rows` (nrows of them)
 * are computed; out is [nrows][N]. */
static int64_t e4m3_times_512(uint8_t c) {
    return (int64_t)(bqo_e4m3_decode(c) * 512.0);
}

void bqo_fp8_acc(const uint8_t* aq, const uint8_t* wq, int64_t M, int64_t N,
                 int64_t K, const int64_t* rows, int64_t nrows, double* out) {
    (void)M;
    int64_t table[256];
    for (int c = 0; c < 256; ++c)
        table[c] = ((c & 0x7F) == 0x7F) ? 0 : e4m3_times_512((uint8_t)c);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        const uint8_t* ar = aq + rows[i] * K;
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* wr = wq + n * K;
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += table[ar[k]] * table[wr[k]];
            out[i * N + n] = ldexp((double)s, -18);
        }
    }
}

/* Y = (sA * sW[n]) * acc, in fp64.  sw has N entries when per_channel,
 * else one. */
void bqo_fp8_linear(const uint8_t* aq, float sa, const uint8_t* wq,
                    const float* sw, int per_channel, int64_t M, int64_t N,
                    int64_t K, const int64_t* rows, int64_t nrows, double* y) {
    bqo_fp8_acc(aq, wq, M, N, K, rows, nrows, y);
    for (int64_t i = 0; i < nrows; ++i)
        for (int64_t n = 0; n < N; ++n)
            y[i * N + n] = (double)sa * (double)sw[per_channel ? n : 0] * y[i * N + n];
}

/* fp8 egress: code = E4M3(Y / output_scale) with the rounding above. */
void bqo_fp8_output(const double* y, int64_t count, float output_scale, uint8_t* codes) {
    for (int64_t i = 0; i < count; ++i)
        codes[i] = bqo_e4m3_encode(y[i] / (double)output_scale);
}

/* Weight-only fp8: Y = sW[n] * sum_k A[m,k] * decode(Wq[n,k]), fp64. */
void bqo_w8a16_linear(const float* a, const uint8_t* wq, const float* sw,
                      int64_t M, int64_t N, int64_t K, const int64_t* rows,
                      int64_t nrows, double* y) {
    (void)M;
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = bqo_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        const float* ar = a + rows[i] * K;
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* wr = wq + n * K;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += (double)ar[k] * table[wr[k]];
            y[i * N + n] = (double)sw[n] * s;
        }
    }
}

/* W4A8: acc[m,n] = sum_k Aq[m,k] * W4[n,k] exactly (int64; the caller
 * checks it fits int32).  The widening of int4 to int8 by *16 and the
 * exact /16 afterwards cancel, so the defining sum is the plain one. */
void bqo_w4a8_acc(const int8_t* aq, const int8_t* w4, int64_t M, int64_t N,
                  int64_t K, const int64_t* rows, int64_t nrows, int64_t* acc) {
    (void)M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        const int8_t* ar = aq + rows[i] * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t* wr = w4 + n * K;
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int64_t)ar[k] * (int64_t)wr[k];
            acc[i * N + n] = s;
        }
    }
}

/* Y = acc * sA[m] * sW[n], fp64. */
void bqo_w4a8_linear(const int64_t* acc, const float* sa, const float* sw,
                     int64_t N, const int64_t* rows, int64_t nrows, double* y) {
    for (int64_t i = 0; i < nrows; ++i)
        for (int64_t n = 0; n < N; ++n)
            y[i * N + n] = (double)acc[i * N + n] * (double)sa[rows[i]] * (double)sw[n];
}

/* ------------------------------------------- RMSNorm ahead of quantization */

/* The QQQ issue #15 answer on online activation quantization says the
 * activation quantizer is fused into an element-wise kernel such as rmsnorm.
 * The pages do not print RMSNorm itself; the standard root-mean-square
 * normalization with eps inside the root is used:
 *   r[m] = 1 / sqrt(mean_k x[m,k]^2 + eps),   y[m,k] = x[m,k] * r[m] * g[k].
 * Precision (our reading, the pages give none): every square of a 16-bit
 * input is exact in fp64 and the squares are summed in fp64; ms = sum / K,
 * ms + eps, the square root and the reciprocal are fp64 operations, and r is
 * that fp64 value rounded once to fp32; y = fp32(fp32(x * r) * g).  The
 * quantizers above are then applied to y unchanged. */

/* Sum of squares of one row, in fp64, in k order. */
double bqo_rms_sumsq(const float* x, int64_t K) {
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += (double)x[k] * (double)x[k];
    return s;
}

/* r = fp32(1 / sqrt(sumsq / K + eps)), each step an fp64 operation. */
float bqo_rms_inv(double sumsq, int64_t K, float eps) {
    double ms = sumsq / (double)K;
    double d = ms + (double)eps;
    double root = sqrt(d);
    return (float)(1.0 / root);
}

/* y[m,k] = fp32(fp32(x[m,k] * r[m]) * g[k]) for given per-row r. */
void bqo_rmsnorm_apply(const float* x, const float* g, const float* r, int64_t M,
                       int64_t K, float* y) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            float t = x[m * K + k] * r[m];
            y[m * K + k] = t * g[k];
        }
}

/* Whole RMSNorm: r (fp32 [M]) from the rows, then y (fp32 [M,K]). */
void bqo_rmsnorm(const float* x, const float* g, int64_t M, int64_t K, float eps,
                 float* y, float* r) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) r[m] = bqo_rms_inv(bqo_rms_sumsq(x + m * K, K), K, eps);
    bqo_rmsnorm_apply(x, g, r, M, K, y);
}

/* ------------------------------------------------- per-group W4A8 (g128) */

/* The QQQ issue #15 tables compare per-channel W4A8 ("qqq") with a per-group
 * variant ("qqq-g128"); the pages name the group size (128) but print no
 * formula.  The plain reading used here: int4 weights with one scale per
 * output channel n and group g of 128 consecutive k, int8 per-token
 * activations, an exact integer sum per group, and the group scales applied
 * to those sums:
 *   acc_g[m,n] = sum_{k in group g} Aq[m,k] * W4[n,k]            (exact)
 *   Y[m,n]     = sA[m] * sum_g sW[n,g] * acc_g[m,n]              (real)
 * computed here in fp64 for the given rows (sW: [N][G] row-major). */
void bqo_w4a8_group_linear(const int8_t* aq, const float* sa, const int8_t* w4, const float* sw,
                           int64_t M, int64_t N, int64_t K, int64_t group, const int64_t* rows,
                           int64_t nrows, double* y) {
    const int64_t G = (K + group - 1) / group;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t m = rows[r];
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                int64_t acc = 0;
                const int64_t k1 = (g + 1) * group < K ? (g + 1) * group : K;
                for (int64_t k = g * group; k < k1; ++k)
                    acc += (int64_t)aq[m * K + k] * (int64_t)w4[n * K + k];
                sum += (double)sw[n * G + g] * (double)acc;
            }
            y[r * N + n] = (double)sa[m] * sum;
        }
    }
    (void)M;
}

/* ------------------------------------------------ per-group W4A16 (g128) */

/* The QQQ issue #15 tables also list weight-only int4 kernels with group
 * size 128 ("awq-g128", "marlin-g128"): 16-bit activations, int4 weights,
 * one scale per output channel and group; the pages give no formula.  The
 * plain reading used here, the same weight format as the per-group W4A8
 * above (two's-complement int4, no zero point):
 *   Y[m,n] = sum_g sW[n,g] * sum_{k in group g} A[m,k] * W4[n,k]
 * with A the fp32 values of the fp16 activations; computed in fp64 for the
 * given rows (sW: [N][G] row-major). */
void bqo_w4a16_group_linear(const float* a, const int8_t* w4, const float* sw, int64_t M,
                            int64_t N, int64_t K, int64_t group, const int64_t* rows,
                            int64_t nrows, double* y) {
    const int64_t G = (K + group - 1) / group;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t m = rows[r];
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                double part = 0.0;
                const int64_t k1 = (g + 1) * group < K ? (g + 1) * group : K;
                for (int64_t k = g * group; k < k1; ++k)
                    part += (double)a[m * K + k] * (double)w4[n * K + k];
                sum += (double)sw[n * G + g] * part;
            }
            y[r * N + n] = sum;
        }
    }
    (void)M;
}
