// RMSNorm fused with the activation quantizers (QQQ issue #15, the answer on
// online activation quantization: the quantizer is fused into an element-wise
// kernel such as rmsnorm, so the normalized activation is never written in
// 16 bits and read back).
//
// RMSNorm is the standard root-mean-square normalization with eps inside the
// root, computed as the library defines it:
//   r[m] = fp32(1 / sqrt(sum_k x[m,k]^2 / K + eps))   (exact squares summed in
//          fp64; the division, the addition, the root and the reciprocal are
//          fp64 operations; one rounding to fp32 at the end),
//   y[m,k] = fp32(fp32(x[m,k] * r[m]) * g[k]).
// The quantizers then act on y exactly as the standalone ones act on x:
//   per-token int8 (QQQ issue #15):     s[m] = amax_m / 127, q = clamp(rne(y / s[m]), +-127);
//   per-tensor E4M3 (vLLM PR #4118):    s = amax / 448,       q = E4M3(y / s);
// with IEEE fp32 divisions y / s, formed as quot_f32 (device.h) forms them.
//
// Kernels.  Grids are persistent (at most 1024 blocks of 256 threads, or 512
// of 1024 threads for K > 8192); a block walks rows gridDim.x apart with
// each row in registers (up to four 16-byte chunks of 8 elements per
// thread), g held for all its rows, and the next row requested before the
// current one is reduced and quantized.  The sum of squares and the row
// maximum are DPP folds within each wave plus a fixed-order fold over the
// block's waves, one barrier each.
// Per-token int8 is one launch.  Per-tensor E4M3 has a grid-wide dependency
// (the amax of y over all rows), so it is two launches: the row kernel
// stores r[m] and the maximum of |y| over each block's rows in the
// workspace, and every block of the cast kernel folds those (at most 1024)
// maxima itself before it re-reads its rows, recomputes y and writes the
// codes.  No atomics, nothing to zero beforehand, and results do not depend
// on the order in which blocks run.
#include "device.h"
#include "kernels.h"

namespace bql {

// Block folds with one barrier (the wave folds are device.h's DPP folds):
// each wave's value goes to sh[wave], then every thread folds sh[0 ..
// BT/64) in order.  A call's writes could race with the reads of the call
// just before it on the same buffer, so consecutive calls in a block must
// use different buffers (any two calls further apart are separated by the
// barrier of the call between them).
template <int BT>
__device__ __forceinline__ double block_sum_1b(double v, double* sh) {
    v = wave_sum_f64(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < BT / 64; ++i) s += sh[i];
    return s;
}

template <int BT>
__device__ __forceinline__ uint32_t block_max_1b(uint32_t v, uint32_t* sh) {
    v = wave_max_u32(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < BT / 64; ++i) m = umax32(m, sh[i]);
    return m;
}

template <int DT>
__device__ __forceinline__ void decode8(const u4& v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = to_f32<DT>(v[j] & 0xFFFFu);
        f[2 * j + 1] = to_f32<DT>(v[j] >> 16);
    }
}

__device__ __forceinline__ uint32_t pack4_i8(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
    return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// Two finite fp32 values -> E4M3 codes (first in bits 0-7): clamp to
// [-448, 448] with med3 (signed zeros pass unchanged), then the nearest-even
// conversion.  The inputs here are finite by contract, so the NaN handling
// of the general encoder is not needed.
__device__ __forceinline__ uint32_t e4m3_encode2_finite(float a, float b) {
    const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ uint32_t int8_code(float q) {
    float t = __builtin_rintf(q);  // ties to even
    t = t > 127.0f ? 127.0f : (t < -127.0f ? -127.0f : t);
    return (uint32_t)(int32_t)t & 0xFFu;
}

// Rows m = blockIdx.x, blockIdx.x + gridDim.x, ... of a block, each held as
// CH 16-byte chunks per thread (chunk c = threadIdx.x + j * BT).  The next
// row is requested before the current one is reduced and quantized, so its
// HBM reads overlap the current row's arithmetic; g stays in registers.
// MODE 0: RMSNorm + per-token int8: q8, scales and (optional) inv_rms.
// MODE 1: first pass of RMSNorm + per-tensor E4M3: r_ws[m] (and inv_rms),
//         and partial[blockIdx.x] = max |y| (fp32 bits) over the block's rows.
template <int DT, int BT, int CH, int MODE>
__global__ __launch_bounds__(BT) void rmsnorm_rows_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ g,
                                                          int64_t M, int64_t K, float eps,
                                                          int8_t* __restrict__ q8,
                                                          float* __restrict__ scales,
                                                          float* __restrict__ inv_rms,
                                                          uint32_t* __restrict__ partial,
                                                          float* __restrict__ r_ws) {
    // per-row sums alternate between two buffers (MODE 1 has no fold in
    // between); MODE 0 alternates the sum with the max, which has its own
    __shared__ double shd[2][BT / 64];
    __shared__ uint32_t shu[BT / 64];
    const int nch = (int)(K / 8);  // K is a multiple of 16
    const u4* gv = (const u4*)g;
    u4 w[CH], v[CH], nx[CH];
    int64_t m = blockIdx.x;
    int parity = 0;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = threadIdx.x + j * BT;
        const u4* row = (const u4*)(x + m * K);
        v[j] = c < nch ? __builtin_nontemporal_load(&row[c]) : u4{0u, 0u, 0u, 0u};
        w[j] = c < nch ? gv[c] : u4{0u, 0u, 0u, 0u};
    }
    uint32_t block_mb = 0;
    for (; m < M; m += gridDim.x) {
        const int64_t mn = m + gridDim.x;
        const u4* nrow = (const u4*)(x + (mn < M ? mn : m) * K);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = threadIdx.x + j * BT;
            nx[j] = (mn < M && c < nch) ? __builtin_nontemporal_load(&nrow[c]) : u4{0u, 0u, 0u, 0u};
        }
        double ss = 0.0;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            float f[8];
            decode8<DT>(v[j], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += (double)f[e] * (double)f[e];  // exact squares
        }
        ss = block_sum_1b<BT>(ss, shd[parity]);
        parity ^= 1;
        const double ms = ss / (double)K;
        const double d = ms + (double)eps;
        const float r = (float)(1.0 / __builtin_sqrt(d));

        float y[CH][8];
        uint32_t mb = 0;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            float f[8], gf[8];
            decode8<DT>(v[j], f);
            decode8<DT>(w[j], gf);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t = f[e] * r;
                y[j][e] = t * gf[e];
                const uint32_t a = __float_as_uint(y[j][e]) & 0x7FFFFFFFu;
                mb = mb > a ? mb : a;
            }
        }
        if constexpr (MODE == 1) {
            block_mb = block_mb > mb ? block_mb : mb;
            if (threadIdx.x == 0) {
                r_ws[m] = r;
                if (inv_rms) inv_rms[m] = r;
            }
        } else {
            mb = block_max_1b<BT>(mb, shu);
            const float amax = __uint_as_float(mb);
            const float s = amax == 0.0f ? 1.0f : amax / 127.0f;  // IEEE division
            const double inv = 1.0 / (double)s;
            u2* out = (u2*)(q8 + m * K);
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int c = threadIdx.x + j * BT;
                if (c < nch) {
                    uint32_t cc[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) cc[e] = int8_code(quot_f32(y[j][e], inv));
                    out[c] = u2{pack4_i8(cc[0], cc[1], cc[2], cc[3]),
                                pack4_i8(cc[4], cc[5], cc[6], cc[7])};
                }
            }
            if (threadIdx.x == 0) {
                scales[m] = s;
                if (inv_rms) inv_rms[m] = r;
            }
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) v[j] = nx[j];
    }
    if constexpr (MODE == 1) {
        block_mb = block_max_1b<BT>(block_mb, shu);
        if (threadIdx.x == 0) partial[blockIdx.x] = block_mb;
    }
}

// Second pass of RMSNorm + per-tensor E4M3: rows m = blockIdx.x,
// + gridDim.x, ... are re-read and cast, each block first folding the
// nparts block maxima of the first pass into the scale.  The first row is
// requested before that fold and each next row before the current one is
// cast.
template <int DT, int BT, int CH>
__global__ __launch_bounds__(BT) void rmsnorm_fp8_cast_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ g, int64_t M, int64_t K,
    const uint32_t* __restrict__ partial, int nparts, const float* __restrict__ r_ws,
    uint8_t* __restrict__ xq, float* __restrict__ scale_out) {
    __shared__ uint32_t shu[BT / 64];
    const int nch = (int)(K / 8);
    const u4* gv = (const u4*)g;
    u4 w[CH], v[CH], nx[CH];
    int64_t m = blockIdx.x;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = threadIdx.x + j * BT;
        const u4* row = (const u4*)(x + m * K);
        v[j] = c < nch ? __builtin_nontemporal_load(&row[c]) : u4{0u, 0u, 0u, 0u};
        w[j] = c < nch ? gv[c] : u4{0u, 0u, 0u, 0u};
    }
    uint32_t mb = 0;
    for (int i = threadIdx.x; i < nparts; i += BT) mb = mb > partial[i] ? mb : partial[i];
    mb = block_max_1b<BT>(mb, shu);  // the block's only fold
    const float amax = __uint_as_float(mb);
    const float s = amax == 0.0f ? 1.0f : amax / 448.0f;  // IEEE division
    const double inv = 1.0 / (double)s;
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
    for (; m < M; m += gridDim.x) {
        const int64_t mn = m + gridDim.x;
        const u4* nrow = (const u4*)(x + (mn < M ? mn : m) * K);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = threadIdx.x + j * BT;
            nx[j] = (mn < M && c < nch) ? __builtin_nontemporal_load(&nrow[c]) : u4{0u, 0u, 0u, 0u};
        }
        const float r = r_ws[m];
        u2* out = (u2*)(xq + m * K);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = threadIdx.x + j * BT;
            if (c < nch) {
                float f[8], gf[8], y[8];
                decode8<DT>(v[j], f);
                decode8<DT>(w[j], gf);
                uint32_t pr[4];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = (f[e] * r) * gf[e];
#pragma unroll
                for (int e = 0; e < 8; e += 2)
                    pr[e / 2] = e4m3_encode2_finite(quot_f32(y[e], inv), quot_f32(y[e + 1], inv));
                __builtin_nontemporal_store(u2{pr[0] | (pr[1] << 16), pr[2] | (pr[3] << 16)}, &out[c]);
            }
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) v[j] = nx[j];
    }
}

size_t rmsnorm_quant_ws_bytes(int64_t M) {
    return (size_t)(((8 * M) + 255) & ~int64_t(255));
}

// Threads per row and chunks per thread: 256 threads with 1, 2 or 4 chunks
// up to K = 8192, then 1024 threads with 2 or 4 chunks up to K = 32768.
// Grids are persistent: at most NQ_BLOCKS_256 (or NQ_BLOCKS_1024) blocks,
// each walking rows gridDim.x apart.
constexpr int64_t NQ_BLOCKS_256 = 1024;
constexpr int64_t NQ_BLOCKS_1024 = 512;

static unsigned nq_grid(int64_t M, int BT) {
    const int64_t cap = BT == 256 ? NQ_BLOCKS_256 : NQ_BLOCKS_1024;
    return (unsigned)(M < cap ? M : cap);
}

template <int DT, int MODE>
static unsigned launch_rows(const void* x, const void* g, int64_t M, int64_t K, float eps,
                            int8_t* q8, float* scales, float* inv_rms, uint32_t* partial,
                            float* r_ws, hipStream_t stream) {
    const uint16_t* xs = (const uint16_t*)x;
    const uint16_t* gs = (const uint16_t*)g;
#define NQ_ROWS(BT, CH)                                                                           \
    do {                                                                                          \
        const unsigned grid = nq_grid(M, BT);                                                     \
        rmsnorm_rows_kernel<DT, BT, CH, MODE><<<grid, BT, 0, stream>>>(xs, gs, M, K, eps, q8,     \
                                                                       scales, inv_rms, partial,  \
                                                                       r_ws);                     \
        return grid;                                                                              \
    } while (0)
    if (K <= 256 * 8) NQ_ROWS(256, 1);
    if (K <= 256 * 16) NQ_ROWS(256, 2);
    if (K <= 256 * 32) NQ_ROWS(256, 4);
    if (K <= 1024 * 16) NQ_ROWS(1024, 2);
    NQ_ROWS(1024, 4);
#undef NQ_ROWS
}

hipError_t launch_rmsnorm_int8(const void* x, const void* g, int xdt, int64_t M, int64_t K,
                               float eps, int8_t* xq, float* scales, float* inv_rms,
                               hipStream_t stream) {
    if (xdt == IN_BF16)
        launch_rows<IN_BF16, 0>(x, g, M, K, eps, xq, scales, inv_rms, nullptr, nullptr, stream);
    else
        launch_rows<IN_F16, 0>(x, g, M, K, eps, xq, scales, inv_rms, nullptr, nullptr, stream);
    return hipGetLastError();
}

template <int DT>
static void launch_fp8(const void* x, const void* g, int64_t M, int64_t K, float eps, uint8_t* xq,
                       float* scale_out, float* inv_rms, void* ws, hipStream_t stream) {
    uint32_t* partial = (uint32_t*)ws;
    float* r_ws = (float*)((char*)ws + 4 * M);
    const uint16_t* xs = (const uint16_t*)x;
    const uint16_t* gs = (const uint16_t*)g;
    const int nparts = (int)launch_rows<DT, 1>(x, g, M, K, eps, nullptr, nullptr, inv_rms, partial,
                                               r_ws, stream);
#define NQ_CAST(BT, CH)                                                                          \
    do {                                                                                         \
        rmsnorm_fp8_cast_kernel<DT, BT, CH><<<nq_grid(M, BT), BT, 0, stream>>>(                  \
            xs, gs, M, K, partial, nparts, r_ws, xq, scale_out);                                 \
        return;                                                                                  \
    } while (0)
    if (K <= 256 * 8) NQ_CAST(256, 1);
    if (K <= 256 * 16) NQ_CAST(256, 2);
    if (K <= 256 * 32) NQ_CAST(256, 4);
    if (K <= 1024 * 16) NQ_CAST(1024, 2);
    NQ_CAST(1024, 4);
#undef NQ_CAST
}

hipError_t launch_rmsnorm_fp8(const void* x, const void* g, int xdt, int64_t M, int64_t K,
                              float eps, uint8_t* xq, float* scale_out, float* inv_rms, void* ws,
                              hipStream_t stream) {
    if (xdt == IN_BF16)
        launch_fp8<IN_BF16>(x, g, M, K, eps, xq, scale_out, inv_rms, ws, stream);
    else
        launch_fp8<IN_F16>(x, g, M, K, eps, xq, scale_out, inv_rms, ws, stream);
    return hipGetLastError();
}

}  // namespace bql
