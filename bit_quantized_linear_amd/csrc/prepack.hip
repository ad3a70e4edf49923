// Weight prepack for gfx950: quantize after load (vLLM PR #4118,
// "Algorithm": per-tensor weight scale computed once and stored with the
// weight; optimum-quanto PR #241: a per-output-channel scale vector) and
// lay the codes out in the MFMA operand order the linear kernels stream.
//
// Layout (see device.h): 16-channel x 128-k tiles, strip-major along k.
// A lane of a wave reads its whole MFMA operand from one tile with
// 16-byte loads, and one wave-wide load instruction covers 1 KiB of
// contiguous memory.  Scales stay in logical channel order; the kernels map
// every accumulator back to its channel n, so a per-channel scale vector
// can never be applied to the wrong column (the interleaving problem raised
// on optimum-quanto PR #241).
#include "device.h"
#include "kernels.h"
#include "skinny.h"

namespace bql {

constexpr int PT = 256;

// scales[n] = amax(W[n, :]) / qmax (1 if the row is all zero), one block per row.
template <int DT>
__global__ __launch_bounds__(PT) void row_scale_kernel(const uint16_t* __restrict__ w, int64_t K,
                                                       float qmax, float* __restrict__ scales) {
    __shared__ uint32_t sh[16];
    const int64_t n = blockIdx.x;
    const uint16_t* row = w + n * K;
    uint32_t m = 0;
    for (int64_t k = threadIdx.x; k < K; k += PT) {
        uint32_t e = mag16(row[k]);
        m = m > e ? m : e;
    }
    m = block_max_u32(m, sh);
    if (threadIdx.x == 0) {
        float amax = to_f32<DT>(m);
        scales[n] = amax == 0.0f ? 1.0f : amax / qmax;
    }
}

// fp16 or fp32 scales -> fp32 (exact).
__global__ void convert_scales_kernel(const void* __restrict__ s, int sdt, int64_t count,
                                      float* __restrict__ out) {
    int64_t i = (int64_t)blockIdx.x * PT + threadIdx.x;
    if (i >= count) return;
    out[i] = sdt == 1 ? to_f32<IN_F16>(((const uint16_t*)s)[i]) : ((const float*)s)[i];
}

// Per-group scales, given [N][G] (fp16 or fp32), stored [G][N] in fp32 so
// that the kernels read one k-tile's scales of consecutive channels together.
__global__ void group_scales_kernel(const void* __restrict__ s, int sdt, int64_t N, int64_t G,
                                    float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * PT + threadIdx.x;  // output index g * N + n
    if (i >= N * G) return;
    const int64_t g = i / N, n = i % N;
    const int64_t src = n * G + g;
    out[i] = sdt == 1 ? to_f32<IN_F16>(((const uint16_t*)s)[src]) : ((const float*)s)[src];
}

// One thread per 16-byte chunk of the packed layout.
template <int SRC>  // IN_F16, IN_BF16, or 4 = E4M3 codes
__global__ __launch_bounds__(PT) void prepack_fp8_kernel(const void* __restrict__ w, int64_t N,
                                                         int64_t K, int64_t KT,
                                                         const float* __restrict__ scales,
                                                         int per_row, uint8_t* __restrict__ packed) {
    const int64_t q = (int64_t)blockIdx.x * PT + threadIdx.x;
    const int64_t total = ((N + TILE_N - 1) / TILE_N) * KT * (FP8_TILE_BYTES / 16);
    if (q >= total) return;
    const int64_t tile = q / (FP8_TILE_BYTES / 16);
    const int c = (int)(q % (FP8_TILE_BYTES / 16));
    const int h = c / 64, lane = c % 64;
    const int64_t nt = tile / KT, kt = tile % KT;
    const int64_t n = nt * TILE_N + (lane & 15);
    const int64_t k0 = kt * TILE_K + 32 * (lane >> 4) + 16 * h;
    uint32_t out[4] = {0, 0, 0, 0};
    // K is a multiple of 16: the chunk is whole or absent; channels past N
    // (only when N < 16) are zero codes
    if (k0 < K && n < N) {
        if constexpr (SRC == 4) {
            const uint32_t* src = (const uint32_t*)((const uint8_t*)w + n * K + k0);
#pragma unroll
            for (int j = 0; j < 4; ++j) out[j] = src[j];
        } else {
            const float s = scales[per_row ? n : 0];
            const uint16_t* src = (const uint16_t*)w + n * K + k0;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                uint32_t code = e4m3_encode(to_f32<SRC>(src[j]) / s);
                out[j >> 2] |= code << (8 * (j & 3));
            }
        }
    }
    u4* dst = (u4*)(packed + tile * FP8_TILE_BYTES + h * 1024 + lane * 16);
    *dst = u4{out[0], out[1], out[2], out[3]};
}

__global__ __launch_bounds__(PT) void unpack_fp8_kernel(const uint8_t* __restrict__ packed,
                                                        int64_t N, int64_t K, int64_t KT,
                                                        uint8_t* __restrict__ out) {
    const int64_t q = (int64_t)blockIdx.x * PT + threadIdx.x;
    const int64_t total = ((N + TILE_N - 1) / TILE_N) * KT * (FP8_TILE_BYTES / 16);
    if (q >= total) return;
    const int64_t tile = q / (FP8_TILE_BYTES / 16);
    const int c = (int)(q % (FP8_TILE_BYTES / 16));
    const int h = c / 64, lane = c % 64;
    const int64_t nt = tile / KT, kt = tile % KT;
    const int64_t n = nt * TILE_N + (lane & 15);
    const int64_t k0 = kt * TILE_K + 32 * (lane >> 4) + 16 * h;
    if (k0 >= K || n >= N) return;
    const u4 v = *(const u4*)(packed + tile * FP8_TILE_BYTES + h * 1024 + lane * 16);
    uint32_t* dst = (uint32_t*)(out + n * K + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = v[j];
}

// Logical int4 (low nibble = even k) -> tiles.  One thread per lane chunk.
__device__ __forceinline__ uint32_t int4_at(const uint8_t* row, int64_t k, int64_t K) {
    if (k >= K) return 0;
    uint8_t b = row[k >> 1];
    return (k & 1) ? (b >> 4) : (b & 15u);
}

__global__ __launch_bounds__(PT) void prepack_int4_kernel(const uint8_t* __restrict__ w, int64_t N,
                                                          int64_t K, int64_t KT,
                                                          uint8_t* __restrict__ packed) {
    const int64_t q = (int64_t)blockIdx.x * PT + threadIdx.x;
    const int64_t total = (N / TILE_N) * KT * 64;
    if (q >= total) return;
    const int64_t tile = q / 64;
    const int lane = (int)(q % 64);
    const int64_t nt = tile / KT, kt = tile % KT;
    const int64_t n = nt * TILE_N + (lane & 15);
    const int64_t k0 = kt * TILE_K + 32 * (lane >> 4);
    const uint8_t* row = w + n * (K / 2);
    uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        uint32_t b = int4_at(row, k0 + j, K) | (int4_at(row, k0 + 16 + j, K) << 4);
        out[j >> 2] |= b << (8 * (j & 3));
    }
    *(u4*)(packed + tile * INT4_TILE_BYTES + lane * 16) = u4{out[0], out[1], out[2], out[3]};
}

__global__ __launch_bounds__(PT) void unpack_int4_kernel(const uint8_t* __restrict__ packed,
                                                         int64_t N, int64_t K, int64_t KT,
                                                         uint8_t* __restrict__ out) {
    // one thread per output byte of the logical layout: k = 2*i, 2*i+1
    const int64_t i = (int64_t)blockIdx.x * PT + threadIdx.x;
    if (i >= N * K / 2) return;
    const int64_t n = (2 * i) / K;
    const int64_t k = (2 * i) % K;
    uint32_t v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int64_t kk = k + e;
        const int64_t kt = kk / TILE_K;
        const int r = (int)(kk % TILE_K);
        const int g = r / 32, j = r % 32;
        const int lane = (int)(n % TILE_N) + 16 * g;
        const uint8_t b = packed[((n / TILE_N) * KT + kt) * INT4_TILE_BYTES + lane * 16 + (j & 15)];
        v[e] = (j < 16) ? (b & 15u) : (b >> 4);
    }
    out[i] = (uint8_t)(v[0] | (v[1] << 4));
}

static unsigned blocks_for(int64_t threads) { return (unsigned)((threads + PT - 1) / PT); }

hipError_t launch_row_scales(const void* w, int wdt, int64_t N, int64_t K, float qmax,
                             float* scales, hipStream_t stream) {
    if (wdt == IN_BF16)
        row_scale_kernel<IN_BF16><<<(unsigned)N, PT, 0, stream>>>((const uint16_t*)w, K, qmax, scales);
    else
        row_scale_kernel<IN_F16><<<(unsigned)N, PT, 0, stream>>>((const uint16_t*)w, K, qmax, scales);
    return hipGetLastError();
}

hipError_t launch_convert_scales(const void* s, int sdt, int64_t count, float* out,
                                 hipStream_t stream) {
    convert_scales_kernel<<<blocks_for(count), PT, 0, stream>>>(s, sdt, count, out);
    return hipGetLastError();
}

hipError_t launch_group_scales(const void* s, int sdt, int64_t N, int64_t G, float* out,
                               hipStream_t stream) {
    group_scales_kernel<<<blocks_for(N * G), PT, 0, stream>>>(s, sdt, N, G, out);
    return hipGetLastError();
}

hipError_t launch_prepack_fp8(const void* w, int wdt, int64_t N, int64_t K, const float* scales,
                              int per_row, uint8_t* packed, hipStream_t stream) {
    const int64_t KT = (K + TILE_K - 1) / TILE_K;
    const unsigned nb = blocks_for(((N + TILE_N - 1) / TILE_N) * KT * (FP8_TILE_BYTES / 16));
    if (wdt == IN_F16)
        prepack_fp8_kernel<IN_F16><<<nb, PT, 0, stream>>>(w, N, K, KT, scales, per_row, packed);
    else if (wdt == IN_BF16)
        prepack_fp8_kernel<IN_BF16><<<nb, PT, 0, stream>>>(w, N, K, KT, scales, per_row, packed);
    else
        prepack_fp8_kernel<4><<<nb, PT, 0, stream>>>(w, N, K, KT, scales, per_row, packed);
    return hipGetLastError();
}

hipError_t launch_prepack_int4(const uint8_t* w, int64_t N, int64_t K, uint8_t* packed,
                               hipStream_t stream) {
    const int64_t KT = (K + TILE_K - 1) / TILE_K;
    prepack_int4_kernel<<<blocks_for((N / TILE_N) * KT * 64), PT, 0, stream>>>(w, N, K, KT, packed);
    return hipGetLastError();
}

hipError_t launch_unpack_fp8(const uint8_t* packed, int64_t N, int64_t K, uint8_t* out,
                             hipStream_t stream) {
    const int64_t KT = (K + TILE_K - 1) / TILE_K;
    unpack_fp8_kernel<<<blocks_for(((N + TILE_N - 1) / TILE_N) * KT * (FP8_TILE_BYTES / 16)), PT, 0, stream>>>(
        packed, N, K, KT, out);
    return hipGetLastError();
}

hipError_t launch_unpack_int4(const uint8_t* packed, int64_t N, int64_t K, uint8_t* out,
                              hipStream_t stream) {
    const int64_t KT = (K + TILE_K - 1) / TILE_K;
    unpack_int4_kernel<<<blocks_for(N * K / 2), PT, 0, stream>>>(packed, N, K, KT, out);
    return hipGetLastError();
}

}  // namespace bql
