// Pieces shared by the linear kernels of the library (small-M streaming,
// LDS-tiled MFMA, and the exact fp8 tile kernel): launch parameters, the
// per-variant operand traits, operand decoding, the epilogue's output
// conversion, and the synchronization and tile-order helpers of the tiled
// kernels.
#pragma once

#include "device.h"
#include "kernels.h"

namespace bql {

struct LinParams {
    const void* a;          // packed 8-bit A (fp8 / int8 variants), row-major 8-bit A (small M,
                            // a_rowmajor), row-major fp16 (W8A16), or row-major fp16/bf16
                            // when the small-M kernel quantizes A itself
    const uint8_t* w;
    int64_t M, N, K, KT;
    int64_t kt_per_split;
    int splits;
    void* partial;
    Epilogue ep;
    int xdt;                // fused quantization: IN_F16 / IN_BF16
    float* scale_out;       // fused quantization: optional copy of sA for the caller
    float* scale_ws;        // fused quantization: sA for the split-K reduce
    int a_rowmajor;         // small-M kernels: 8-bit A is row-major [M, K], not packed
    const float* given_scale;  // fused quantization with a static scale (no amax) when set
};

template <int V> struct VT;
template <> struct VT<V_FP8> {
    static constexpr int B_TILE = FP8_TILE_BYTES;
    static constexpr int A_CHUNKS = 2;  // 16-byte chunks of A per lane per k-tile
    static constexpr int B_CHUNKS = 2;
    using Acc = v4f;
    using E = float;
};
template <> struct VT<V_FP8X> {
    static constexpr int B_TILE = FP8_TILE_BYTES;
    static constexpr int A_CHUNKS = 2;
    static constexpr int B_CHUNKS = 2;
    using Acc = v4f;
    using E = float;
};
template <> struct VT<V_W8A16> {
    static constexpr int B_TILE = FP8_TILE_BYTES;
    static constexpr int A_CHUNKS = 4;
    static constexpr int B_CHUNKS = 2;
    using Acc = v4f;
    using E = float;
};
template <> struct VT<V_W4A8> {
    static constexpr int B_TILE = INT4_TILE_BYTES;
    static constexpr int A_CHUNKS = 2;
    static constexpr int B_CHUNKS = 1;
    using Acc = v4i;
    using E = int;
};
// Per-group W4A8: the B operand of the small-M kernels carries the k-tile's
// group scale of the lane's channel as a second chunk (x component).
// Per-group W4A16: fp16 A as W8A16, the int4 tile and the k-tile's group
// scale as V_W4A8G.
template <> struct VT<V_W4A16G> {
    static constexpr int B_TILE = INT4_TILE_BYTES;
    static constexpr int A_CHUNKS = 4;
    static constexpr int B_CHUNKS = 2;
    using Acc = v4f;
    using E = float;
};
template <> struct VT<V_W4A8G> {
    static constexpr int B_TILE = INT4_TILE_BYTES;
    static constexpr int A_CHUNKS = 2;
    static constexpr int B_CHUNKS = 2;
    using Acc = v4f;
    using E = float;
};

__device__ __forceinline__ v8i as_v8i(const u4& x0, const u4& x1) {
    return v8i{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
               (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
}

__device__ __forceinline__ v4i as_v4i(const u4& x) {
    return v4i{(int)x[0], (int)x[1], (int)x[2], (int)x[3]};
}

// A lane's 32 E4M3 codes (k0 .. k0+31) as four fp16 operands of 8.
__device__ __forceinline__ void decode32(const u4& x0, const u4& x1, v8h (&h)[4]) {
    h[0] = e4m3x8_to_f16(x0[0], x0[1]);
    h[1] = e4m3x8_to_f16(x0[2], x0[3]);
    h[2] = e4m3x8_to_f16(x1[0], x1[1]);
    h[3] = e4m3x8_to_f16(x1[2], x1[3]);
}

__device__ __forceinline__ void mma_w4a8(v4i& acc, const u4& alo, const u4& ahi, const u4& b) {
    const v4i blo = {(int)int4_lo_x16(b[0]), (int)int4_lo_x16(b[1]),
                     (int)int4_lo_x16(b[2]), (int)int4_lo_x16(b[3])};
    const v4i bhi = {(int)int4_hi_x16(b[0]), (int)int4_hi_x16(b[1]),
                     (int)int4_hi_x16(b[2]), (int)int4_hi_x16(b[3])};
    acc = mfma_i8(as_v4i(alo), blo, acc);
    acc = mfma_i8(as_v4i(ahi), bhi, acc);
}

// One k-tile of per-group W4A8: the exact int32 sum of the tile (a 128-k
// group, of 16 * W4 products) times s16 = group scale / 16, added in fp32.
// |t| < 2^24 converts exactly, and s16 is exact wherever the scale is a
// normal float above 2^-122, so each term is the single rounding of
// (t / 16) * scale.  Two VALU instructions per accumulator per group, which
// at the chip's rates already cost as much as the group's MFMAs.
__device__ __forceinline__ void group_fold(v4f& acc, const u4& alo, const u4& ahi, const u4& b,
                                           float s16) {
    v4i t = v4i{0, 0, 0, 0};
    mma_w4a8(t, alo, ahi, b);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf((float)t[r], s16, acc[r]);
}

template <int V>
__device__ __forceinline__ void mma(typename VT<V>::Acc& acc, const u4 (&a)[VT<V>::A_CHUNKS],
                                    const u4 (&b)[VT<V>::B_CHUNKS]) {
    if constexpr (V == V_FP8) {
        acc = mfma_fp8(as_v8i(a[0], a[1]), as_v8i(b[0], b[1]), acc);
    } else if constexpr (V == V_W4A8) {
        mma_w4a8(acc, a[0], a[1], b[0]);
    } else if constexpr (V == V_W4A8G) {
        group_fold(acc, a[0], a[1], b[0], __uint_as_float(b[1][0]) * 0.0625f);
    } else if constexpr (V == V_W4A16G) {
        // the k-tile is one 128-k group: its sum over the f16 matrix cores
        // (exact products), then times the group scale into fp32
        const uint32_t d[4] = {b[0][0], b[0][1], b[0][2], b[0][3]};
        v8h bh[4];
        int4x32_to_f16(d, bh);
        v4f t = v4f{0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) t = mfma_f16(__builtin_bit_cast(v8h, a[q]), bh[q], t);
        const float s = __uint_as_float(b[1][0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(t[r], s, acc[r]);
    } else if constexpr (V == V_FP8X) {
        // four f16 MFMAs over k0+8q .. k0+8q+7 on losslessly decoded codes
        v8h ah[4], bh[4];
        decode32(a[0], a[1], ah);
        decode32(b[0], b[1], bh);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = mfma_f16(ah[q], bh[q], acc);
    } else {  // W8A16: A is fp16 already
        v8h bh[4];
        decode32(b[0], b[1], bh);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = mfma_f16(__builtin_bit_cast(v8h, a[q]), bh[q], acc);
    }
}

template <int V>
__device__ __forceinline__ void finish(const LinParams& p, float sa, int64_t m, int64_t n,
                                       typename VT<V>::E v) {
    if constexpr (V == V_W4A8) epilogue_int(p.ep, m, n, v);
    else if constexpr (V == V_W4A8G) store_out(p.ep, m, n, v * p.ep.a_scale[m]);
    else if constexpr (V == V_W4A16G) store_out(p.ep, m, n, v);
    else epilogue_float(p.ep, sa, m, n, v);
}

// Output value of one accumulator as the output dtype's bits (same
// arithmetic as epilogue_float / epilogue_int).
template <int V>
__device__ __forceinline__ uint32_t out_bits(const Epilogue& ep, float sa, int64_t m, int64_t n,
                                             typename VT<V>::E v) {
    float y;
    if constexpr (V == V_W4A8) {
        const int acc = v >> 4;
        if (ep.ydt == OUT_I32) return (uint32_t)acc;
        y = ((float)acc * ep.a_scale[m]) * ep.w_scale[n];
    } else if constexpr (V == V_W4A8G) {
        y = v * ep.a_scale[m];
    } else if constexpr (V == V_W4A16G) {
        y = v;
    } else {
        y = (sa * ep.w_scale[ep.w_per_channel ? n : 0]) * v;
    }
    if (ep.ydt == OUT_F16) return f32_to_f16_bits(y);
    if (ep.ydt == OUT_BF16) return f32_to_bf16_bits(y);
    if (ep.ydt == OUT_F32) return __float_as_uint(y);
    return e4m3_encode2(y / *ep.out_scale, 0.0f) & 0xFFu;
}

__device__ __forceinline__ int out_size(int ydt) {
    return ydt == OUT_E4M3 ? 1 : ((ydt == OUT_F32 || ydt == OUT_I32) ? 4 : 2);
}

// s_waitcnt vmcnt(N) that leaves the other counters alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup barrier that orders LDS accesses only. __syncthreads() also
// drains every outstanding global load (vmcnt 0), which would retire the
// LDS-DMA stages still in flight behind the one being waited for; the
// DMA stages are waited for explicitly with wait_vmcnt instead.
__device__ __forceinline__ void lds_barrier() {
    // lgkmcnt(0): this wave's LDS reads have returned (vmcnt, expcnt left open)
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_s_barrier();
}

// Output tile of hardware block b. Blocks are dispatched to the 8 XCDs in
// turn (block b to XCD b % 8) and each XCD has its own L2, so each XCD is
// given one contiguous range of tiles; within it tiles run in groups of
// GROUP_M tile rows, row index fastest, so that the blocks resident at the
// same time on an XCD share A and W strips (read once into its L2, then hit).
constexpr int XCDS = 8, GROUP_M = 8;
__device__ __forceinline__ void tile_coords(int64_t b, int64_t nbm, int64_t nbn, int64_t& bm, int64_t& bn) {
    const int64_t tiles = nbm * nbn, q = tiles / XCDS, r = tiles % XCDS;
    const int64_t x = b % XCDS, j = b / XCDS;
    const int64_t t = x * q + (x < r ? x : r) + j;
    const int64_t group = t / (GROUP_M * nbn), first = group * GROUP_M;
    const int64_t gm = nbm - first < GROUP_M ? nbm - first : GROUP_M;
    const int64_t rem = t - group * GROUP_M * nbn;
    bm = first + rem % gm;
    bn = rem / gm;
}

// The exact fp8 tile kernel (256-row blocks of four waves of 128 rows, or
// eight of 64 rows, each by fn 16-column strips); defined in gemm_exact.hip.  exact_plan gives its
// block width (fn 0: the kernel is not used at this shape) and K splits;
// launch_gemm_exact takes p.splits and p.kt_per_split as planned.
struct ExactPlan {
    int fn;
    int splits;
};
ExactPlan exact_plan(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_exact(const LinParams& p, const ExactPlan& plan, hipStream_t stream);

// Launch of the per-group W4A16 tile kernel (128-row blocks of 256 or 128
// columns, four waves side by side in N); defined in gemm_w4a16.hip.
// w4a16_tile_fits tells whether a shape is inside that kernel's offset
// range; w4a16_plan gives the block width (fn 16-channel strips per wave)
// and K splits (fp32 partials in the workspace, then the split-K reduce).
struct W4A16Plan {
    int fn;
    int splits;
};
W4A16Plan w4a16_plan(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_w4a16(const LinParams& p, hipStream_t stream);
bool w4a16_tile_fits(int64_t M, int64_t N, int64_t K);
int w4a16_tile_splits(int64_t M, int64_t N, int64_t K);

}  // namespace bql
