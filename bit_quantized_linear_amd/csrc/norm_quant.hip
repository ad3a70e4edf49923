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
// with IEEE fp32 divisions (y is an arbitrary fp32 value here, so the
// reciprocal shortcut of the 16-bit quantizers does not apply).
//
// Kernels.  A block owns a row and keeps it in registers (at most 4 chunks of
// 8 elements per thread, so 256 threads cover K <= 8192 and 1024 threads
// K <= 32768); the sum of squares and the row maximum are wave shuffles plus
// a fixed-order fold over the block's waves.  Per-token int8 is one launch.
// Per-tensor E4M3 has a grid-wide dependency (the amax of y over all rows),
// so it is two launches: the row kernel stores r[m] and max_k |y[m,k]| in the
// workspace, and every block of the cast kernel folds the M row maxima
// itself before it re-reads its rows, recomputes y and writes the codes.  No
// atomics, nothing to zero beforehand, and results do not depend on the
// order in which blocks run.
#include "device.h"
#include "kernels.h"

namespace bql {

constexpr int NQ_CHUNKS = 4;        // 16-byte chunks per thread in the row kernel
constexpr int NQ_CAST_T = 256;      // threads per block of the cast kernel
constexpr int NQ_CAST_BLOCKS = 1024;

// Sum over the block in a fixed order, returned to every thread.
// `sh` holds >= 16 doubles.
__device__ __forceinline__ double block_sum_f64(double v, double* sh) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = (blockDim.x + 63) >> 6;
    __syncthreads();
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    double s = 0.0;
    for (int i = 0; i < nw; ++i) s += sh[i];
    return s;
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

// MODE 0: RMSNorm + per-token int8, writes q8, scales and (optional) inv_rms.
// MODE 1: first pass of RMSNorm + per-tensor E4M3: writes r_ws[m], the row
//         maximum of |y| (as fp32 bits) to rowmax[m], and optional inv_rms.
template <int DT, int BT, int MODE>
__global__ __launch_bounds__(BT) void rmsnorm_rows_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ g,
                                                          int64_t K, float eps,
                                                          int8_t* __restrict__ q8,
                                                          float* __restrict__ scales,
                                                          float* __restrict__ inv_rms,
                                                          uint32_t* __restrict__ rowmax,
                                                          float* __restrict__ r_ws) {
    __shared__ double shd[16];
    __shared__ uint32_t shu[16];
    const int64_t m = blockIdx.x;
    const int nch = (int)(K / 8);  // K is a multiple of 16
    const u4* row = (const u4*)(x + m * K);
    const u4* gv = (const u4*)g;
    u4 v[NQ_CHUNKS];
#pragma unroll
    for (int j = 0; j < NQ_CHUNKS; ++j) {
        const int c = threadIdx.x + j * BT;
        v[j] = c < nch ? __builtin_nontemporal_load(&row[c]) : u4{0u, 0u, 0u, 0u};
    }
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < NQ_CHUNKS; ++j) {
        float f[8];
        decode8<DT>(v[j], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += (double)f[e] * (double)f[e];  // exact squares
    }
    ss = block_sum_f64(ss, shd);
    const double ms = ss / (double)K;
    const double d = ms + (double)eps;
    const float r = (float)(1.0 / __builtin_sqrt(d));

    float y[NQ_CHUNKS][8];
    uint32_t mb = 0;
#pragma unroll
    for (int j = 0; j < NQ_CHUNKS; ++j) {
        const int c = threadIdx.x + j * BT;
        const u4 w = c < nch ? gv[c] : u4{0u, 0u, 0u, 0u};
        float f[8], gf[8];
        decode8<DT>(v[j], f);
        decode8<DT>(w, gf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float t = f[e] * r;
            y[j][e] = t * gf[e];
            const uint32_t a = __float_as_uint(y[j][e]) & 0x7FFFFFFFu;
            mb = mb > a ? mb : a;
        }
    }
    mb = block_max_u32(mb, shu);
    if constexpr (MODE == 1) {
        if (threadIdx.x == 0) {
            rowmax[m] = mb;
            r_ws[m] = r;
            if (inv_rms) inv_rms[m] = r;
        }
    } else {
        const float amax = __uint_as_float(mb);
        const float s = amax == 0.0f ? 1.0f : amax / 127.0f;  // IEEE division
        u2* out = (u2*)(q8 + m * K);
#pragma unroll
        for (int j = 0; j < NQ_CHUNKS; ++j) {
            const int c = threadIdx.x + j * BT;
            if (c < nch) {
                uint32_t cc[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float t = __builtin_rintf(y[j][e] / s);  // IEEE division, ties to even
                    t = t > 127.0f ? 127.0f : (t < -127.0f ? -127.0f : t);
                    cc[e] = (uint32_t)(int32_t)t & 0xFFu;
                }
                out[c] = u2{pack4_i8(cc[0], cc[1], cc[2], cc[3]), pack4_i8(cc[4], cc[5], cc[6], cc[7])};
            }
        }
        if (threadIdx.x == 0) {
            scales[m] = s;
            if (inv_rms) inv_rms[m] = r;
        }
    }
}

// Second pass of RMSNorm + per-tensor E4M3: fold the row maxima into the
// scale, then rows [blockIdx.x * rpb, +rpb) are re-read and cast.
template <int DT>
__global__ __launch_bounds__(NQ_CAST_T) void rmsnorm_fp8_cast_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ g, int64_t M, int64_t K,
    const uint32_t* __restrict__ rowmax, const float* __restrict__ r_ws, int64_t rpb,
    uint8_t* __restrict__ xq, float* __restrict__ scale_out) {
    __shared__ uint32_t shu[16];
    uint32_t mb = 0;
    for (int64_t i = threadIdx.x; i < M; i += NQ_CAST_T) mb = mb > rowmax[i] ? mb : rowmax[i];
    mb = block_max_u32(mb, shu);
    const float amax = __uint_as_float(mb);
    const float s = amax == 0.0f ? 1.0f : amax / 448.0f;  // IEEE division
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
    const int nch = (int)(K / 8);
    const u4* gv = (const u4*)g;
    const int64_t m0 = (int64_t)blockIdx.x * rpb;
    for (int64_t m = m0; m < m0 + rpb && m < M; ++m) {
        const float r = r_ws[m];
        const u4* row = (const u4*)(x + m * K);
        u2* out = (u2*)(xq + m * K);
        for (int c = threadIdx.x; c < nch; c += NQ_CAST_T) {
            float f[8], gf[8];
            decode8<DT>(__builtin_nontemporal_load(&row[c]), f);
            decode8<DT>(gv[c], gf);
            uint32_t pr[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float y0 = (f[e] * r) * gf[e];
                const float y1 = (f[e + 1] * r) * gf[e + 1];
                pr[e / 2] = e4m3_encode2(y0 / s, y1 / s);  // IEEE divisions
            }
            __builtin_nontemporal_store(u2{pr[0] | (pr[1] << 16), pr[2] | (pr[3] << 16)}, &out[c]);
        }
    }
}

size_t rmsnorm_quant_ws_bytes(int64_t M) {
    return (size_t)(((8 * M) + 255) & ~int64_t(255));
}

template <int DT, int MODE>
static void launch_rows(const void* x, const void* g, int64_t M, int64_t K, float eps, int8_t* q8,
                        float* scales, float* inv_rms, uint32_t* rowmax, float* r_ws,
                        hipStream_t stream) {
    if (K <= 256 * NQ_CHUNKS * 8)
        rmsnorm_rows_kernel<DT, 256, MODE><<<(unsigned)M, 256, 0, stream>>>(
            (const uint16_t*)x, (const uint16_t*)g, K, eps, q8, scales, inv_rms, rowmax, r_ws);
    else
        rmsnorm_rows_kernel<DT, 1024, MODE><<<(unsigned)M, 1024, 0, stream>>>(
            (const uint16_t*)x, (const uint16_t*)g, K, eps, q8, scales, inv_rms, rowmax, r_ws);
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

hipError_t launch_rmsnorm_fp8(const void* x, const void* g, int xdt, int64_t M, int64_t K,
                              float eps, uint8_t* xq, float* scale_out, float* inv_rms, void* ws,
                              hipStream_t stream) {
    uint32_t* rowmax = (uint32_t*)ws;
    float* r_ws = (float*)((char*)ws + 4 * M);
    const int64_t blocks = M < NQ_CAST_BLOCKS ? M : NQ_CAST_BLOCKS;
    const int64_t rpb = (M + blocks - 1) / blocks;
    const int64_t grid = (M + rpb - 1) / rpb;
    if (xdt == IN_BF16) {
        launch_rows<IN_BF16, 1>(x, g, M, K, eps, nullptr, nullptr, inv_rms, rowmax, r_ws, stream);
        rmsnorm_fp8_cast_kernel<IN_BF16><<<(unsigned)grid, NQ_CAST_T, 0, stream>>>(
            (const uint16_t*)x, (const uint16_t*)g, M, K, rowmax, r_ws, rpb, xq, scale_out);
    } else {
        launch_rows<IN_F16, 1>(x, g, M, K, eps, nullptr, nullptr, inv_rms, rowmax, r_ws, stream);
        rmsnorm_fp8_cast_kernel<IN_F16><<<(unsigned)grid, NQ_CAST_T, 0, stream>>>(
            (const uint16_t*)x, (const uint16_t*)g, M, K, rowmax, r_ws, rpb, xq, scale_out);
    }
    return hipGetLastError();
}

}  // namespace bql
