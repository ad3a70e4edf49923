// Activation quantizers for gfx950.
//
// Per-tensor dynamic E4M3 (vLLM PR #4118, "Algorithm": a new activation
// scale every forward pass): scale = amax / 448, codes = E4M3(x / scale)
// with an IEEE fp32 division, nearest-even rounding and saturation.  The
// amax is a grid-wide dependency, so it takes two launches: per-block
// partial maxima, then a cast kernel in which every block first folds the
// (at most 1024) partials itself.  No atomics, no counters, nothing to
// zero beforehand, and the result does not depend on the launch order.
//
// Per-token int8 for the W4A8 activations (QQQ issue #15, the answer on
// online activation quantization): one block per row.
#include "device.h"
#include "kernels.h"
#include "skinny.h"

namespace bql {

constexpr int QT = 256;          // threads per block
constexpr int MAX_PARTIALS = 1024;  // fills the 4 KiB partials region of the workspace
constexpr int AMAX_LOADS = 8;       // 16-byte loads in flight per thread

int amax_blocks(int64_t numel) {
    int64_t vecs = (numel + 7) / 8;
    int64_t b = (vecs + QT * AMAX_LOADS - 1) / (QT * AMAX_LOADS);
    if (b < 1) b = 1;
    if (b > MAX_PARTIALS) b = MAX_PARTIALS;
    return (int)b;
}

// Each block: max of |x| (as ordered magnitude bits) over a grid-stride
// range of 16-byte vectors, AMAX_LOADS loads in flight per thread; the
// scalar tail (numel % 8) goes to block 0.
__global__ __launch_bounds__(QT) void amax_partial_kernel(const uint16_t* __restrict__ x,
                                                          int64_t numel,
                                                          uint32_t* __restrict__ partial) {
    __shared__ uint32_t sh[16];
    const int64_t nvec = numel / 8;
    const u4* xv = (const u4*)x;
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * QT;
    int64_t i = (int64_t)blockIdx.x * QT + threadIdx.x;
    auto fold = [&](const u4& v) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = mag16(v[j] & 0xFFFFu), hi = mag16(v[j] >> 16);
            m = m > lo ? m : lo;
            m = m > hi ? m : hi;
        }
    };
    for (; i + (AMAX_LOADS - 1) * stride < nvec; i += AMAX_LOADS * stride) {
        u4 v[AMAX_LOADS];
#pragma unroll
        for (int u = 0; u < AMAX_LOADS; ++u) v[u] = __builtin_nontemporal_load(&xv[i + u * stride]);
#pragma unroll
        for (int u = 0; u < AMAX_LOADS; ++u) fold(v[u]);
    }
    for (; i < nvec; i += stride) fold(__builtin_nontemporal_load(&xv[i]));
    if (blockIdx.x == 0) {
        int64_t t = nvec * 8 + threadIdx.x;
        if (t < numel) {
            uint32_t e = mag16(x[t]);
            m = m > e ? m : e;
        }
    }
    m = block_max_u32(m, sh);
    if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

template <int DT>
__device__ __forceinline__ float scale_from_partials(const uint32_t* partial, int nparts,
                                                     float qmax, uint32_t* sh) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += blockDim.x) m = m > partial[i] ? m : partial[i];
    m = block_max_u32(m, sh);
    float amax = to_f32<DT>(m);
    return amax == 0.0f ? 1.0f : amax / qmax;  // IEEE division
}

__device__ __forceinline__ uint32_t pack4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
    return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// Cast kernel.  SCALE_FROM: 0 = fold amax partials, 1 = read a given scale.
template <int DT, int SCALE_FROM>
__global__ __launch_bounds__(QT) void cast_e4m3_kernel(const uint16_t* __restrict__ x,
                                                       int64_t numel,
                                                       const uint32_t* __restrict__ partial,
                                                       int nparts,
                                                       const float* __restrict__ given,
                                                       uint8_t* __restrict__ xq,
                                                       float* __restrict__ scale_out,
                                                       float* __restrict__ scale_ws) {
    __shared__ uint32_t sh[16];
    float s;
    if constexpr (SCALE_FROM == 0) {
        s = scale_from_partials<DT>(partial, nparts, 448.0f, sh);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            if (scale_out) *scale_out = s;
            if (scale_ws) *scale_ws = s;
        }
    } else {
        s = *given;
    }
    const int64_t nvec = numel / 8;
    const u4* xv = (const u4*)x;
    u2* qv = (u2*)xq;
    // enc2(a, b): the code pair of a / s and b / s
    auto body = [&](auto enc2) {
        for (int64_t i = (int64_t)blockIdx.x * QT + threadIdx.x; i < nvec;
             i += (int64_t)gridDim.x * QT) {
            u4 v = xv[i];  // plain load: x was just read by the amax pass
            uint32_t c[4];  // code pairs
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = enc2(to_f32<DT>(v[j] & 0xFFFFu), to_f32<DT>(v[j] >> 16));
            u2 o = {c[0] | (c[1] << 16), c[2] | (c[3] << 16)};
            __builtin_nontemporal_store(o, &qv[i]);
        }
        if (blockIdx.x == 0) {
            int64_t t = nvec * 8 + threadIdx.x;
            if (t < numel) xq[t] = (uint8_t)(enc2(to_f32<DT>(x[t]), 0.0f) & 0xFFu);
        }
    };
    // a given (static) scale is any float: only the dynamic scale amax/448
    // takes the reciprocal form
    const float y = 1.0f / s;
    if (SCALE_FROM == 0 && recip_div_ok(s))
        body([&](float a, float b) { return e4m3_div2_finite(a, b, s, y); });
    else
        body([&](float a, float b) { return e4m3_encode2(a / s, b / s); });
}

// ------------------------------------------------ packed 8-bit activations
//
// The linear kernels read 8-bit activations in the MFMA operand tile layout
// the weights use: tiles of 16 rows x 128 k (2048 B), all k-tiles of a
// 16-row strip consecutive, a tile stored as [half h][lane l][16 B] with
// row l % 16 and k = 32*(l/16) + 16*h + j.  Columns k >= K up to the tile
// edge and rows past M in the last strip hold zero codes.

// One wave's inputs of packed tile t (16 rows x 128 k).  Rows past M and k
// past K (K is a multiple of 16) read as zero; every load is issued (from a
// valid address when out of range) so that none sits in a branch.  Plain
// loads, not nontemporal ones: the amax pass has just read x, and plain
// loads find more of it still cached (the Llama-3-8B fp8 step at M = 1024
// is 0.7 % faster).  Loads cover whole lines of 4 rows each, and each
// lane stores its codes where the operand layout puts them (the layout's
// own lane map as the load map touches 16 rows in 16-byte pieces per
// instruction: the step 0.6 % slower).
struct TileIn {
    u4 v[4];
};

// Row-contiguous loads: load q of lane L takes row 4q + L/16 of the tile,
// inputs k = 128 kt + 8 (L%16) .. +7 (whole 128-byte lines per instruction).
__device__ __forceinline__ void load_tile_in(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                             int64_t KT, int64_t t, int r, int g, TileIn& in) {
    const int lane = r + 16 * g;
    const int64_t mt = t / KT, kt = t % KT;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t m = mt * 16 + 4 * q + (lane >> 4), k = kt * 128 + 8 * (lane & 15);
        const bool ok = m < M && k < K;
        const u4 v = *(const u4*)(ok ? x + m * K + k : x);
        in.v[q] = ok ? v : u4{0u, 0u, 0u, 0u};
    }
}

// The 8 codes of each load go to their place in the operand tile: row rr,
// k = 8 c .. lies in lane rr + 16 (c / 4), half (c % 4) / 2, bytes 8 (c % 2).
template <int DT, class Enc>
__device__ __forceinline__ void store_tile_codes(const TileIn& in, uint8_t* __restrict__ xq,
                                                 int64_t t, int lane, Enc enc2) {
    const int c = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int rr = 4 * q + (lane >> 4);
        const u4& v = in.v[q];
        uint32_t p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = enc2(to_f32<DT>(v[j] & 0xFFFFu), to_f32<DT>(v[j] >> 16));
        uint8_t* dst = xq + t * 2048 + ((c & 3) >> 1) * 1024 + (rr + 16 * (c >> 2)) * 16 + 8 * (c & 1);
        *(u2*)dst = u2{p[0] | (p[1] << 16), p[2] | (p[3] << 16)};
    }
}

// The tile loop of the packed casts, for a given encoder enc2(a, b) of the
// code pair of a / s and b / s: wave w of block b takes tiles t0 = b * WPB +
// w, t0 + gridDim.x * WPB, ...; the inputs of t0 were requested by the
// caller before it had the scale (`first`).
template <int DT, class Enc>
__device__ __forceinline__ void cast_packed_tiles(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                  int64_t KT, uint8_t* __restrict__ xq, int64_t tiles,
                                                  int lane, int r, int g, const TileIn& first, Enc enc2) {
    constexpr int WPB = QT / 64;
    const int64_t stride = (int64_t)gridDim.x * WPB;
    int64_t t = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
    if (t >= tiles) return;
    store_tile_codes<DT>(first, xq, t, lane, enc2);
    for (t += stride; t < tiles; t += stride) {
        TileIn in;
        load_tile_in(x, M, K, KT, t, r, g, in);
        store_tile_codes<DT>(in, xq, t, lane, enc2);
    }
}

// Blocks of the packed casts: one tile per wave up to 8192 blocks (more
// waves in flight measured faster than fewer waves that each prefetch their
// next tile).
static int64_t packed_cast_blocks(int64_t tiles) {
    const int64_t blocks = (tiles + QT / 64 - 1) / (QT / 64);
    return blocks < 8192 ? blocks : 8192;
}

// One wave per 16 x 128 packed tile (row tile mt, k-tile kt), grid-stride
// over tiles. Lane l = r + 16 g holds row 16 mt + r, k = 128 kt + 32 g ..
// +31: it reads those 32 inputs (64 contiguous bytes; a row's four lanes read
// 256 contiguous bytes) and writes the 16 codes of k .. k+15 at tile + 16 l
// and those of k+16 .. k+31 at tile + 1024 + 16 l, so each wave stores two
// contiguous 1 KiB runs. Rows past M and k past K (K is a multiple of 16)
// are written as zero codes.
template <int DT>
__global__ __launch_bounds__(QT) void cast_e4m3_packed_kernel(const uint16_t* __restrict__ x,
                                                              int64_t M, int64_t K, int64_t KT,
                                                              const uint32_t* __restrict__ partial,
                                                              int nparts, uint8_t* __restrict__ xq,
                                                              float* __restrict__ scale_out,
                                                              float* __restrict__ scale_ws) {
    __shared__ uint32_t sh[16];
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int64_t tiles = ((M + 15) / 16) * KT;
    // the first tile's inputs are requested before the partials are folded,
    // so their HBM latency overlaps the fold's
    const int64_t t0 = (int64_t)blockIdx.x * (QT / 64) + (threadIdx.x >> 6);
    TileIn first;
    load_tile_in(x, M, K, KT, t0 < tiles ? t0 : 0, r, g, first);
    const float s = scale_from_partials<DT>(partial, nparts, 448.0f, sh);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (scale_out) *scale_out = s;
        if (scale_ws) *scale_ws = s;
    }
    const float y = 1.0f / s;
    if (recip_div_ok(s))
        cast_packed_tiles<DT>(x, M, K, KT, xq, tiles, lane, r, g, first,
                              [&](float a, float b) { return e4m3_div2_finite(a, b, s, y); });
    else
        cast_packed_tiles<DT>(x, M, K, KT, xq, tiles, lane, r, g, first,
                              [&](float a, float b) { return e4m3_encode2(a / s, b / s); });
}

// Static-scale cast into the packed layout: s is given (checkpoint
// input_scale, or a scale kept from an earlier call), so there is no amax
// pass; x / s is the IEEE quotient formed by quot_f32.
template <int DT>
__global__ __launch_bounds__(QT) void cast_e4m3_packed_static_kernel(const uint16_t* __restrict__ x,
                                                                     int64_t M, int64_t K, int64_t KT,
                                                                     const float* __restrict__ given,
                                                                     uint8_t* __restrict__ xq) {
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int64_t tiles = ((M + 15) / 16) * KT;
    const int64_t t0 = (int64_t)blockIdx.x * (QT / 64) + (threadIdx.x >> 6);
    TileIn first;
    load_tile_in(x, M, K, KT, t0 < tiles ? t0 : 0, r, g, first);
    const double inv = 1.0 / (double)*given;
    cast_packed_tiles<DT>(x, M, K, KT, xq, tiles, lane, r, g, first, [&](float a, float b) {
        return e4m3_encode2(quot_f32(a, inv), quot_f32(b, inv));
    });
}

// Row-major 8-bit codes [M, K] -> packed layout: one wave per 16 x 128
// tile (grid-stride), lane l = r + 16 g moving row 16 mt + r, k = 128 kt +
// 32 g .. +31 (two 16-byte loads) to tile + 16 l and tile + 1024 + 16 l, so
// each wave reads 128 contiguous bytes per row and stores two contiguous
// 1 KiB runs. Rows past M and k past K (a multiple of 16) become zero codes.
__global__ __launch_bounds__(QT) void pack_codes_kernel(const uint8_t* __restrict__ src, int64_t M,
                                                        int64_t K, int64_t KT,
                                                        uint8_t* __restrict__ dst) {
    constexpr int WPB = QT / 64;
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int64_t tiles = ((M + 15) / 16) * KT;
    for (int64_t t = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6); t < tiles;
         t += (int64_t)gridDim.x * WPB) {
        const int64_t m = (t / KT) * 16 + r, k = (t % KT) * 128 + 32 * g;
        const bool row = m < M;
        const u4 lo = row && k < K ? *(const u4*)(src + m * K + k) : u4{0, 0, 0, 0};
        const u4 hi = row && k + 16 < K ? *(const u4*)(src + m * K + k + 16) : u4{0, 0, 0, 0};
        uint8_t* tile = dst + t * 2048 + lane * 16;
        *(u4*)tile = lo;
        *(u4*)(tile + 1024) = hi;
    }
}

size_t packed_act_bytes(int64_t M, int64_t K) {
    return (size_t)((M + 15) / 16) * (size_t)((K + 127) / 128) * 2048;
}

hipError_t launch_quant_dynamic_packed(const void* x, int xdt, int64_t M, int64_t K, uint8_t* xq,
                                       float* scale_out, void* ws, hipStream_t stream) {
    uint32_t* partial = (uint32_t*)ws;
    float* scale_ws = (float*)((char*)ws + 4096);
    const int64_t numel = M * K;
    const int nb = amax_blocks(numel);
    amax_partial_kernel<<<nb, QT, 0, stream>>>((const uint16_t*)x, numel, partial);
    const int64_t KT = (K + 127) / 128;
    const int64_t blocks = packed_cast_blocks(((M + 15) / 16) * KT);
    if (xdt == IN_BF16)
        cast_e4m3_packed_kernel<IN_BF16><<<(unsigned)blocks, QT, 0, stream>>>(
            (const uint16_t*)x, M, K, KT, partial, nb, xq, scale_out, scale_ws);
    else
        cast_e4m3_packed_kernel<IN_F16><<<(unsigned)blocks, QT, 0, stream>>>(
            (const uint16_t*)x, M, K, KT, partial, nb, xq, scale_out, scale_ws);
    return hipGetLastError();
}

hipError_t launch_pack_codes(const uint8_t* src, int64_t M, int64_t K, uint8_t* dst,
                             hipStream_t stream) {
    const int64_t KT = (K + 127) / 128;
    int64_t blocks = (((M + 15) / 16) * KT + QT / 64 - 1) / (QT / 64);
    if (blocks > 8192) blocks = 8192;
    pack_codes_kernel<<<(unsigned)blocks, QT, 0, stream>>>(src, M, K, KT, dst);
    return hipGetLastError();
}

// scale = amax / qmax over a whole tensor, for weight prepack.
template <int DT>
__global__ __launch_bounds__(QT) void finalize_scale_kernel(const uint32_t* __restrict__ partial,
                                                            int nparts, float qmax,
                                                            float* __restrict__ scale) {
    __shared__ uint32_t sh[16];
    float s = scale_from_partials<DT>(partial, nparts, qmax, sh);
    if (threadIdx.x == 0) *scale = s;
}

static int cast_blocks(int64_t numel) {
    int64_t vecs = (numel + 7) / 8;
    int64_t b = (vecs + QT - 1) / QT;
    if (b < 1) b = 1;
    if (b > 8192) b = 8192;
    return (int)b;
}

hipError_t launch_quant_dynamic(const void* x, int xdt, int64_t numel, uint8_t* xq,
                                float* scale_out, void* ws, hipStream_t stream) {
    uint32_t* partial = (uint32_t*)ws;
    float* scale_ws = (float*)((char*)ws + 4096);
    const int nb = amax_blocks(numel);
    amax_partial_kernel<<<nb, QT, 0, stream>>>((const uint16_t*)x, numel, partial);
    if (xdt == IN_BF16)
        cast_e4m3_kernel<IN_BF16, 0><<<cast_blocks(numel), QT, 0, stream>>>(
            (const uint16_t*)x, numel, partial, nb, nullptr, xq, scale_out, scale_ws);
    else
        cast_e4m3_kernel<IN_F16, 0><<<cast_blocks(numel), QT, 0, stream>>>(
            (const uint16_t*)x, numel, partial, nb, nullptr, xq, scale_out, scale_ws);
    return hipGetLastError();
}

hipError_t launch_quant_static(const void* x, int xdt, int64_t numel, const float* scale,
                               uint8_t* xq, hipStream_t stream) {
    if (xdt == IN_BF16)
        cast_e4m3_kernel<IN_BF16, 1><<<cast_blocks(numel), QT, 0, stream>>>(
            (const uint16_t*)x, numel, nullptr, 0, scale, xq, nullptr, nullptr);
    else
        cast_e4m3_kernel<IN_F16, 1><<<cast_blocks(numel), QT, 0, stream>>>(
            (const uint16_t*)x, numel, nullptr, 0, scale, xq, nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_quant_static_packed(const void* x, int xdt, int64_t M, int64_t K,
                                      const float* scale, uint8_t* xq, hipStream_t stream) {
    const int64_t KT = (K + 127) / 128;
    const int64_t blocks = packed_cast_blocks(((M + 15) / 16) * KT);
    if (xdt == IN_BF16)
        cast_e4m3_packed_static_kernel<IN_BF16><<<(unsigned)blocks, QT, 0, stream>>>(
            (const uint16_t*)x, M, K, KT, scale, xq);
    else
        cast_e4m3_packed_static_kernel<IN_F16><<<(unsigned)blocks, QT, 0, stream>>>(
            (const uint16_t*)x, M, K, KT, scale, xq);
    return hipGetLastError();
}

int launch_amax_partials(const void* x, int64_t numel, uint32_t* partial, hipStream_t stream) {
    const int nb = amax_blocks(numel);
    amax_partial_kernel<<<nb, QT, 0, stream>>>((const uint16_t*)x, numel, partial);
    return nb;
}

hipError_t launch_tensor_scale(const void* x, int xdt, int64_t numel, float qmax,
                               float* scale, void* ws, hipStream_t stream) {
    uint32_t* partial = (uint32_t*)ws;
    const int nb = amax_blocks(numel);
    amax_partial_kernel<<<nb, QT, 0, stream>>>((const uint16_t*)x, numel, partial);
    if (xdt == IN_BF16)
        finalize_scale_kernel<IN_BF16><<<1, QT, 0, stream>>>(partial, nb, qmax, scale);
    else
        finalize_scale_kernel<IN_F16><<<1, QT, 0, stream>>>(partial, nb, qmax, scale);
    return hipGetLastError();
}

// ------------------------------------------------------- per-token int8

template <int DT>
__global__ __launch_bounds__(QT) void int8_per_token_kernel(const uint16_t* __restrict__ x,
                                                            int64_t K,
                                                            int8_t* __restrict__ xq,
                                                            float* __restrict__ scales) {
    __shared__ uint32_t sh[16];
    const int64_t m = blockIdx.x;
    const u4* row = (const u4*)(x + m * K);
    const int64_t nvec = K / 8;  // K is a multiple of 16
    uint32_t mb = 0;
    for (int64_t i = threadIdx.x; i < nvec; i += QT) {
        u4 v = row[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t lo = mag16(v[j] & 0xFFFFu), hi = mag16(v[j] >> 16);
            mb = mb > lo ? mb : lo;
            mb = mb > hi ? mb : hi;
        }
    }
    mb = block_max_u32(mb, sh);
    const float amax = to_f32<DT>(mb);
    const float s = amax == 0.0f ? 1.0f : amax / 127.0f;
    if (threadIdx.x == 0) scales[m] = s;
    u2* out = (u2*)(xq + m * K);
    for (int64_t i = threadIdx.x; i < nvec; i += QT) {
        u4 v = row[i];
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t b = (j & 1) ? (v[j >> 1] >> 16) : (v[j >> 1] & 0xFFFFu);
            float t = __builtin_rintf(to_f32<DT>(b) / s);
            t = t > 127.0f ? 127.0f : (t < -127.0f ? -127.0f : t);
            c[j] = (uint32_t)(int32_t)t & 0xFFu;
        }
        out[i] = u2{pack4(c[0], c[1], c[2], c[3]), pack4(c[4], c[5], c[6], c[7])};
    }
}

hipError_t launch_int8_per_token(const void* x, int xdt, int64_t M, int64_t K, int8_t* xq,
                                 float* scales, hipStream_t stream) {
    if (xdt == IN_BF16)
        int8_per_token_kernel<IN_BF16><<<(unsigned)M, QT, 0, stream>>>((const uint16_t*)x, K, xq,
                                                                        scales);
    else
        int8_per_token_kernel<IN_F16><<<(unsigned)M, QT, 0, stream>>>((const uint16_t*)x, K, xq,
                                                                       scales);
    return hipGetLastError();
}

}  // namespace bql
