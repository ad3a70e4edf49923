// Device-side helpers shared by the gfx950 kernels of the library.
//
// E4M3 here is the OCP FP8 E4M3 format named by the vLLM FP8
// quantization-schema RFC (Scope): bias 7, three mantissa bits, no
// infinity, S.1111.111 = NaN, largest finite 448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bql {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

enum InDtype { IN_F16 = 1, IN_BF16 = 2 };
enum OutDtype { OUT_F16 = 1, OUT_BF16 = 2, OUT_F32 = 3, OUT_E4M3 = 4, OUT_I32 = 6 };

// Packed-weight tiles: 16 output channels x 128 k.  FP8 tiles hold 2048
// bytes as [half h][lane l][16 bytes]; lane l covers channel l % 16 and
// k = 32*(l/16) + 16*h + j.  INT4 tiles hold 1024 bytes as [lane][16 bytes];
// byte j of lane l has k = 32*(l/16) + j in its low nibble and k + 16 in its
// high nibble.  Tiles of one 16-channel strip are consecutive along k.
constexpr int TILE_N = 16;
constexpr int TILE_K = 128;
constexpr int FP8_TILE_BYTES = 2048;
constexpr int INT4_TILE_BYTES = 1024;

// ----------------------------------------------------------- conversions

template <int DT>
__device__ __forceinline__ float to_f32(uint32_t bits16) {
    if constexpr (DT == IN_BF16) {
        return __uint_as_float(bits16 << 16);
    } else {
        _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
        return (float)h;
    }
}

// |x| as an integer that orders like |x| (non-NaN), for an exact amax.
__device__ __forceinline__ uint32_t mag16(uint32_t bits16) { return bits16 & 0x7FFFu; }

// fp32 -> bf16, nearest with ties to even, on gfx950's v_cvt_pk_bf16_f32
// (one instruction per pair; it equals the bit-level rounding
// (u + 0x7FFF + lsb) >> 16 on every non-NaN fp32 pattern, and keeps NaNs
// NaN, which that formula does not for every payload).
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lo, hi}, v2bf16));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return f32x2_to_bf16x2(f, 0.0f) & 0xFFFFu;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    _Float16 h = (_Float16)f;  // v_cvt_f16_f32: nearest, ties to even
    return __builtin_bit_cast(uint16_t, h);
}

// x / s for the dynamic per-tensor quantizers, from y = 1/s (computed once
// with an IEEE division) and one fma residual correction:
// q = x*y, r = x - q*s (exact), q' = q + r*y, sign taken from x (s > 0).
// For every scale s = amax/448 with amax a finite bf16 or f16 value and
// 2^-90 <= s <= 2^90, and every x of the same format with |x| <= amax, this
// is the IEEE quotient x/s bit for bit wherever |x/s| >= 2^-10; below that
// (tiny x, whose residual may underflow) both quotients stay below 2^-10
// with the sign of x, so both encode to the same signed zero (checked by
// enumerating all such pairs).
// Callers use the IEEE division for scales outside that range.
__device__ __forceinline__ bool recip_div_ok(float s) { return s >= 0x1p-90f && s <= 0x1p90f; }
__device__ __forceinline__ float div_by_scale(float x, float s, float y) {
    const float q = x * y;
    const float r = __builtin_fmaf(-q, s, x);
    return __builtin_copysignf(__builtin_fmaf(r, y, q), x);
}

// The IEEE fp32 quotient y / s of a finite fp32 y by a finite s > 0, from
// inv = 1/s rounded to fp64 (one fp64 division, hoisted by the caller):
// p = y * inv in fp64 is within 2^-52 of y / s (relative).  The rounding
// boundaries of fp32 are the midpoints between neighbouring fp32 values; an
// exact quotient y / s is never one of them in the normal range (a midpoint
// has a 25-bit odd significand, and y = m * s would give y an odd part of at
// least 25 bits), and when it is not, y - m*s is a non-zero multiple of
// 2^(e_m + e_s - 47), which keeps y / s at least 2^-49 (relative) from every
// boundary.  So p rounds to the same fp32 value as y / s.  Below the fp32
// normal range both are tiny values of the sign of y, whose quantization
// codes are zero either way.  gfx950 runs fp64 multiplies and conversions
// at the fp32 rate: three instructions instead of the IEEE division's
// eleven, one of which is a quarter-rate reciprocal.
__device__ __forceinline__ float quot_f32(float y, double inv) {
    return (float)((double)y * inv);
}

// fp32 -> OCP E4M3 code: round to nearest even on the bit pattern,
// saturate magnitudes >= 448 to 0x7E, keep the sign (so -0 -> 0x80).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    // Branch-free (both candidates computed, then selected): the quantizers
    // encode 16-32 values per lane, and data-dependent branches diverge.
    const uint32_t u = __float_as_uint(v);
    const uint32_t s = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    // |v| < 2^-6: subnormal grid of 2^-9, exact scaling then ties-to-even;
    // the input is clamped so the conversion stays in range (t <= 8)
    const float t = __uint_as_float(a < 0x3C800000u ? a : 0x3C800000u) * 512.0f;
    const uint32_t sub = (uint32_t)__builtin_rintf(t);
    // normal: keep 3 of 23 mantissa bits with ties to even, carry into the
    // exponent, then rebias the exponent from 127 to 7 (120 << 3 = 960)
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    const uint32_t nrm = (r >> 20) - 960u;
    uint32_t c = a < 0x3C800000u ? sub : nrm;
    c = a >= 0x43E00000u ? 0x7Eu : c;  // |v| >= 448 (and inf) saturate
    c = a > 0x7F800000u ? 0x7Fu : c;   // NaN
    return s | c;
}

// Two fp32 -> OCP E4M3 codes (a in bits 0-7, b in bits 8-15), the same codes
// as e4m3_encode, with the gfx950 conversion instruction: the input is first
// clamped to [-448, 448] with med3 (infinities saturate, zero keeps its sign;
// a NaN becomes 448, which takes the NaN's sign back from copysign), the
// conversion rounds to nearest even, and a NaN input then gets its low code
// bit set (0x7E -> 0x7F, 0xFE -> 0xFF).  Compared with e4m3_encode on every
// fp32 bit pattern in both positions.
__device__ __forceinline__ uint32_t e4m3_encode2(float a, float b) {
    const float ca = __builtin_copysignf(__builtin_amdgcn_fmed3f(a, -448.0f, 448.0f), a);
    const float cb = __builtin_copysignf(__builtin_amdgcn_fmed3f(b, -448.0f, 448.0f), b);
    const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
    return c | (a != a ? 1u : 0u) | (b != b ? 0x100u : 0u);
}

// A data type as a compile-time argument of a generic lambda.
template <int D>
struct DtTag {
    static constexpr int value = D;
};

// E4M3 codes of xa / s and xb / s (first in bits 0-7) for finite xa, xb:
// the quotient as div_by_scale forms it (y = 1/s), clamped to [-448, 448]
// with med3 and given the sign of x, then the nearest-even conversion.  For
// finite inputs these are the codes of e4m3_encode2(div_by_scale(xa, s, y),
// div_by_scale(xb, s, y)) with three instructions per value fewer (one sign
// transfer and the NaN test).  The dynamic quantizers take it only where
// recip_div_ok(s) holds: s = amax / 448 is then finite, and a NaN or an
// infinity anywhere in the tensor would have made amax non-finite.
__device__ __forceinline__ uint32_t e4m3_div2_finite(float xa, float xb, float s, float y) {
    auto quot = [&](float x) {
        const float q = x * y;
        return __builtin_fmaf(__builtin_fmaf(-q, s, x), y, q);
    };
    const float ca = __builtin_copysignf(__builtin_amdgcn_fmed3f(quot(xa), -448.0f, 448.0f), xa);
    const float cb = __builtin_copysignf(__builtin_amdgcn_fmed3f(quot(xb), -448.0f, 448.0f), xb);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
}

// ------------------------------------------------------------- reductions
//
// Wave folds use DPP lane moves inside each 16-lane row: quad_perm
// [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.  At every
// step a lane and its partner combine the same two values, so after the
// four steps every lane of a row holds the row's fold (max is symmetric and
// an IEEE sum is commutative, so partners agree bit for bit).  The four
// rows are then combined from lanes 0, 16, 32, 48 in a fixed order, giving
// a value that is uniform over the wave, with no LDS round trip.  All 64
// lanes must be active.

constexpr int DPP_QP_1032 = 0xB1, DPP_QP_2301 = 0x4E, DPP_ROW_HALF_MIRROR = 0x141,
              DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = dpp_u32<CTRL>((uint32_t)b), hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
    return __longlong_as_double((long long)((hi << 32) | lo));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __longlong_as_double((long long)((hi << 32) | lo));
}

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = umax32(v, dpp_u32<DPP_QP_1032>(v));
    v = umax32(v, dpp_u32<DPP_QP_2301>(v));
    v = umax32(v, dpp_u32<DPP_ROW_HALF_MIRROR>(v));
    v = umax32(v, dpp_u32<DPP_ROW_MIRROR>(v));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return umax32(umax32(r0, r1), umax32(r2, r3));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_f64<DPP_QP_1032>(v);
    v += dpp_f64<DPP_QP_2301>(v);
    v += dpp_f64<DPP_ROW_HALF_MIRROR>(v);
    v += dpp_f64<DPP_ROW_MIRROR>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Max over the block, returned to every thread: each wave's max goes to
// sh[wave], one barrier, then every thread folds sh in order.  `sh` holds
// >= 16 words.  With a single barrier, two folds through the same buffer
// need a barrier of their own between them (every caller here folds
// through its buffer once per kernel, or alternates buffers).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* sh) {
    v = wave_max_u32(v);
    const int nw = (blockDim.x + 63) >> 6;
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t m = 0;
    for (int i = 0; i < nw; ++i) m = umax32(m, sh[i]);
    return m;
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
    // scale operands of 0 select the unscaled v_mfma_f32_16x16x128_f8f6f4;
    // format 0 for both operands is E4M3
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4i mfma_i8(const v4i& a, const v4i& b, const v4i& c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_f16(const v8h& a, const v8h& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Eight E4M3 codes (two dwords, bytes in k order) -> eight fp16 with the
// same values.  Every finite E4M3 value (|v| <= 448, subnormals down to
// 2^-9) is an fp16 value, so v_cvt_scalef32_pk_f16_fp8 with scale 1.0 is
// lossless; fp16 x fp16 products are exact in the fp32 matrix-core sum.
__device__ __forceinline__ v8h e4m3x8_to_f16(uint32_t d0, uint32_t d1) {
    v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)d0, 1.0f, false);
    v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)d0, 1.0f, true);
    v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)d1, 1.0f, false);
    v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)d1, 1.0f, true);
    return v8h{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Four int4 values (the low nibbles of a dword's bytes, k in byte order) ->
// four fp16 of the same values, two per dword.  Each nibble n (two's
// complement) becomes n ^ 8 in 0..15; a byte permute places it under the
// exponent byte 0x64, which is the fp16 value 1024 + (n ^ 8), and one packed
// fp16 subtraction of 1032 leaves n exactly.
__device__ __forceinline__ void int4x4_to_f16(uint32_t nibbles, uint32_t& lo, uint32_t& hi) {
    const uint32_t x = (nibbles & 0x0F0F0F0Fu) ^ 0x08080808u;
    // v_perm_b32 selectors: 0-3 pick bytes of x, 4 a byte of 0x64646464
    const v2h l = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u));
    const v2h h = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u));
    lo = __builtin_bit_cast(uint32_t, l - v2h{(_Float16)1032.0f, (_Float16)1032.0f});
    hi = __builtin_bit_cast(uint32_t, h - v2h{(_Float16)1032.0f, (_Float16)1032.0f});
}

// A lane's 16 packed int4 bytes (32 values: byte j holds k = k0 + j in its
// low nibble and k0 + 16 + j in its high nibble) -> four fp16 operands of
// 8 consecutive k: k0 .. k0+7, k0+8 .., k0+16 .., k0+24 ...
__device__ __forceinline__ void int4x32_to_f16(const uint32_t (&d)[4], v8h (&h)[4]) {
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int4x4_to_f16(d[i], w[2 * i], w[2 * i + 1]);            // low nibbles: k0 + 4i ..
        int4x4_to_f16(d[i] >> 4, w[8 + 2 * i], w[8 + 2 * i + 1]);  // high nibbles: k0 + 16 + 4i ..
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        h[q] = __builtin_bit_cast(v8h, v4i{(int)w[4 * q], (int)w[4 * q + 1], (int)w[4 * q + 2], (int)w[4 * q + 3]});
}

// Sixteen int4 values (one dword pair of a lane's packed bytes) -> int8
// operands multiplied by 16: low nibbles shifted up, high nibbles masked.
__device__ __forceinline__ uint32_t int4_lo_x16(uint32_t d) { return (d << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t int4_hi_x16(uint32_t d) { return d & 0xF0F0F0F0u; }

// ------------------------------------------------------------- epilogue

struct Epilogue {
    void* y;                 // [M, N] output
    int64_t ldy;             // row stride of y in elements
    int ydt;                 // OutDtype
    const float* a_scale;    // fp8: one sA; w4a8: sA[M]; w8a16: unused
    const float* w_scale;    // sW[0] or sW[N]
    int w_per_channel;
    const float* out_scale;  // E4M3 output only
};

__device__ __forceinline__ void store_out(const Epilogue& ep, int64_t m, int64_t n, float v) {
    if (ep.ydt == OUT_F16) {
        ((uint16_t*)ep.y)[m * ep.ldy + n] = (uint16_t)f32_to_f16_bits(v);
    } else if (ep.ydt == OUT_BF16) {
        ((uint16_t*)ep.y)[m * ep.ldy + n] = (uint16_t)f32_to_bf16_bits(v);
    } else if (ep.ydt == OUT_F32) {
        ((float*)ep.y)[m * ep.ldy + n] = v;
    } else {  // OUT_E4M3
        float t = v / *ep.out_scale;
        ((uint8_t*)ep.y)[m * ep.ldy + n] = (uint8_t)e4m3_encode(t);
    }
}

// Y = (sA * sW[n]) * acc for the fp8 linear; sW[n] * acc for W8A16 (sA = 1).
__device__ __forceinline__ void epilogue_float(const Epilogue& ep, float sa, int64_t m, int64_t n, float acc) {
    float sw = ep.w_scale[ep.w_per_channel ? n : 0];
    float s = sa * sw;
    store_out(ep, m, n, s * acc);
}

// W4A8: acc16 = sum Aq * (16 W4); acc = acc16 / 16 (exact); Y = (acc*sA[m])*sW[n].
__device__ __forceinline__ void epilogue_int(const Epilogue& ep, int64_t m, int64_t n, int acc16) {
    int acc = acc16 >> 4;
    if (ep.ydt == OUT_I32) {
        ((int32_t*)ep.y)[m * ep.ldy + n] = acc;
        return;
    }
    float v = ((float)acc * ep.a_scale[m]) * ep.w_scale[n];
    store_out(ep, m, n, v);
}

}  // namespace bql
