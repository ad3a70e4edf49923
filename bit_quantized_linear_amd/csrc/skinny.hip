// Small-N fp8 linear: the MoE router shape of the vLLM FP8 quantization-
// schema RFC discussion (gate_proj with 8 experts, which FP8 GEMMs that need
// N divisible by 16 leave in 16-bit).  N < 16 needs no padding in memory
// beyond the weight's own 16-channel strip (a few KiB): the 16-wide matrix
// core tile is padded in registers only.  The work is bound by reading A
// once (2*M*N*K flops over M*K bytes of codes, or 2*M*K of fp16/bf16), so
// the idle MFMA columns cost nothing that matters.
//
// A block of 8 waves owns one 16-row strip of A; wave w multiplies k-tiles
// w, w + 8, ... in batches of two, with two register sets used in turn: the
// next batch is requested before the current one is cast and multiplied,
// and the first batch before the activation scale is read.  A lane's 32 operand bytes of a
// 16 x 128 tile are 32 consecutive k of one row (row = lane % 16, k =
// 32 * (lane / 16) + 0..31, the packed layout's lane map).  A is read where
// it is, row-major, by loads that each cover whole lines of a few rows, and
// regrouped into that lane map through a small LDS area per wave: E4M3
// codes as they are, fp16 / bf16 then cast to codes in registers (no packed
// copy of A is written).  The W tile comes from the
// single weight strip, which stays in L2.  The 8 partial 16x16 accumulators
// are summed through LDS in a fixed order and wave 0 applies the epilogue
// to the N real columns.
#include "skinny.h"

namespace bql {

constexpr int SK_WAVES = 8;
constexpr int SK_BATCH = 2;  // k-tiles per register set (two sets alternate)
constexpr int SRC_CODES = 4;

// A lane's share of one 16 x 128 tile of A: two 16-byte chunks of E4M3
// codes, or four of fp16 / bf16.
template <int SRC>
struct ARaw {
    static constexpr int N = SRC == 4 ? 2 : 4;
    u4 v[N];
};

// Row-contiguous loads of one 16 x 128 tile of A (columns k0 ..): codes as
// two loads where lane L takes row 8q + L/8, chunk L%8; fp16 / bf16 as four
// loads where lane L takes row 4q + L/16, chunk L%16.  Each instruction
// reads whole 128-byte lines (the operand layout's own lane map would touch
// 16 rows in 16-byte pieces per instruction: the dynamic router call 7 %
// slower).  Rows past M and chunks past K (a multiple of 16) read as zero.
// Plain loads: with a dynamic scale the amax pass has just read A, and
// plain loads find more of it cached than nontemporal ones (8 %).
template <int SRC>
__device__ __forceinline__ void load_a_rows(const void* a, int64_t M, int64_t K, int64_t mt, int64_t k0,
                                            int lane, ARaw<SRC>& r) {
    constexpr int ES = SRC == 4 ? 1 : 2;
    constexpr int LPR = SRC == 4 ? 8 : 16;   // lanes per row
    constexpr int RPI = 64 / LPR;            // rows per instruction
    constexpr int STEP = 16 / ES;            // elements per chunk
    const uint8_t* base = (const uint8_t*)a;
#pragma unroll
    for (int q = 0; q < ARaw<SRC>::N; ++q) {
        const int64_t m = mt * 16 + RPI * q + lane / LPR;
        const int64_t k = k0 + STEP * (lane % LPR);
        const bool ok = m < M && k < K;
        const u4 v = *(const u4*)(ok ? base + (m * K + k) * ES : base);
        r.v[q] = ok ? v : u4{0u, 0u, 0u, 0u};
    }
}

// Regroups a row-contiguous tile into the operand layout (lane (r, g) holds
// row r, k 32 g .. 32 g + 31) through the wave's own 16 LDS rows (one
// 16-byte pad per row).  LDS instructions of one wave execute in order, so
// each wait only orders the compiler's code and hands the read data over;
// the wave's next tile overwrites the rows only after these reads.
template <int SRC>
__device__ __forceinline__ void to_operand(ARaw<SRC>& r, u4* lds, int lane) {
    constexpr int LPR = SRC == 4 ? 8 : 16;
    constexpr int RPI = 64 / LPR;
    constexpr int RS = LPR + 1;  // u4 per LDS row (one pad)
    constexpr int NQ = ARaw<SRC>::N;
#pragma unroll
    for (int q = 0; q < NQ; ++q) lds[(RPI * q + lane / LPR) * RS + lane % LPR] = r.v[q];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < NQ; ++j) r.v[j] = lds[(lane & 15) * RS + NQ * (lane >> 4) + j];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// The lane's 32 codes of one k-tile as two 16-byte halves: codes as loaded,
// or fp16 / bf16 cast as E4M3(x / sA), enc2(a, b) giving the code pair.
template <int SRC, class Enc>
__device__ __forceinline__ void codes_a(const ARaw<SRC>& r, Enc enc2, u4 (&out)[2]) {
    if constexpr (SRC == 4) {
        out[0] = r.v[0];
        out[1] = r.v[1];
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t c[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u4& v = r.v[2 * h + j / 2];
                const uint32_t d0 = v[2 * (j & 1)], d1 = v[2 * (j & 1) + 1];
                const uint32_t lo = enc2(to_f32<SRC>(d0 & 0xFFFFu), to_f32<SRC>(d0 >> 16));
                const uint32_t hi = enc2(to_f32<SRC>(d1 & 0xFFFFu), to_f32<SRC>(d1 >> 16));
                c[j] = lo | (hi << 16);
            }
            out[h] = u4{c[0], c[1], c[2], c[3]};
        }
    }
}

template <int SRC, bool FAST>
__global__ __launch_bounds__(64 * SK_WAVES) void skinny_linear_kernel(
    const void* __restrict__ a, const uint8_t* __restrict__ w, int64_t M, int64_t N, int64_t K,
    int64_t KT, const float* __restrict__ scale, const uint32_t* __restrict__ partial, int nparts,
    float* __restrict__ scale_out, Epilogue ep) {
    __shared__ v4f red[SK_WAVES][64];
    __shared__ uint32_t sh[16];
    __shared__ u4 lds_a[SK_WAVES][16 * 17];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t mt = blockIdx.x;
    const uint8_t* wt = w + lane * 16;
    ARaw<SRC> ra[SK_BATCH], rb[SK_BATCH];
    u4 wa[SK_BATCH][2], wb[SK_BATCH][2];
    auto load_batch = [&](int64_t kt0, ARaw<SRC> (&raw)[SK_BATCH], u4 (&bv)[SK_BATCH][2]) {
#pragma unroll
        for (int u = 0; u < SK_BATCH; ++u) {
            const int64_t kt = kt0 + u * SK_WAVES;
            const int64_t kv = kt < KT ? kt : 0;  // past K: a valid tile, multiplied by zero A
            load_a_rows<SRC>(a, M, K, mt, kt * TILE_K, lane, raw[u]);
#pragma unroll
            for (int h = 0; h < 2; ++h) bv[u][h] = *(const u4*)(wt + kv * FP8_TILE_BYTES + h * 1024);
        }
    };
    // The first batch is requested before the scale is read or folded, so
    // the scale's latency hides under it.
    constexpr int64_t STEP = SK_WAVES * SK_BATCH;
    load_batch(wave, ra, wa);
    float sa;
    if (nparts > 0) {  // uniform: dynamic scale from the amax partials
        uint32_t mb = 0;
        for (int i = threadIdx.x; i < nparts; i += 64 * SK_WAVES) mb = mb > partial[i] ? mb : partial[i];
        mb = block_max_u32(mb, sh);
        const float amax = to_f32<SRC == SRC_CODES ? IN_F16 : SRC>(mb);
        sa = amax == 0.0f ? 1.0f : amax / 448.0f;  // IEEE division, as the standalone quantizer
        if (blockIdx.x == 0 && threadIdx.x == 0 && scale_out) *scale_out = sa;
    } else {
        sa = *scale;
    }
    v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // The main loop for a given encoder enc2(a, b) of the code pair of
    // a / sA and b / sA.
    auto main_loop = [&](auto enc2) __attribute__((always_inline)) {
        auto compute = [&](const ARaw<SRC> (&raw)[SK_BATCH], const u4 (&bv)[SK_BATCH][2]) {
#pragma unroll
            for (int u = 0; u < SK_BATCH; ++u) {
                u4 av[2];
                ARaw<SRC> t = raw[u];
                to_operand<SRC>(t, lds_a[wave], lane);
                codes_a<SRC>(t, enc2, av);
                if constexpr (FAST) {
                    const v8i x = v8i{(int)av[0][0], (int)av[0][1], (int)av[0][2], (int)av[0][3],
                                      (int)av[1][0], (int)av[1][1], (int)av[1][2], (int)av[1][3]};
                    const v8i y = v8i{(int)bv[u][0][0], (int)bv[u][0][1], (int)bv[u][0][2], (int)bv[u][0][3],
                                      (int)bv[u][1][0], (int)bv[u][1][1], (int)bv[u][1][2], (int)bv[u][1][3]};
                    acc = mfma_fp8(x, y, acc);
                } else {
                    // the lane's 32 codes of each operand, 8 at a time, widened
                    // losslessly to fp16: four 16x16x32 products per k-tile
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        acc = mfma_f16(e4m3x8_to_f16(av[h][0], av[h][1]),
                                       e4m3x8_to_f16(bv[u][h][0], bv[u][h][1]), acc);
                        acc = mfma_f16(e4m3x8_to_f16(av[h][2], av[h][3]),
                                       e4m3x8_to_f16(bv[u][h][2], bv[u][h][3]), acc);
                    }
                }
            }
        };
        // Two batches per trip, the sets swapping roles without copies; a batch
        // past K reads zero A and adds nothing.  The sched barriers keep each
        // batch's loads ahead of the casts and multiplies before them (the
        // scheduler would otherwise sink them behind waits).
        for (int64_t kt = wave; kt < KT; kt += 2 * STEP) {
            load_batch(kt + STEP, rb, wb);
            __builtin_amdgcn_sched_barrier(0);
            compute(ra, wa);
            if (kt + STEP >= KT) break;  // this wave has no second batch
            load_batch(kt + 2 * STEP, ra, wa);
            __builtin_amdgcn_sched_barrier(0);
            compute(rb, wb);
        }
    };
    // A dynamic scale (amax / 448 of this tensor, so every input is finite
    // when the scale passes its range check) takes the reciprocal form and
    // the encoder without NaN handling, as the standalone quantizer; a given
    // scale the fp64-reciprocal IEEE quotient.
    if (nparts > 0 && recip_div_ok(sa)) {
        const float y = 1.0f / sa;
        main_loop([&](float p0, float p1) { return e4m3_div2_finite(p0, p1, sa, y); });
    } else {
        const double inv = 1.0 / (double)sa;
        main_loop([&](float p0, float p1) { return e4m3_encode2(quot_f32(p0, inv), quot_f32(p1, inv)); });
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    v4f sum = red[0][lane];
#pragma unroll
    for (int i = 1; i < SK_WAVES; ++i) {
        const v4f t = red[i][lane];
        sum = v4f{sum[0] + t[0], sum[1] + t[1], sum[2] + t[2], sum[3] + t[3]};
    }
    // C[4 * (lane / 16) + i][lane % 16]: row of the strip, channel
    const int64_t n = lane & 15;
    if (n >= N) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t mo = mt * TILE_N + 4 * (lane >> 4) + i;
        if (mo < M) epilogue_float(ep, sa, mo, n, sum[i]);
    }
}

hipError_t launch_skinny_linear(const void* a, int adt, const uint8_t* w, int64_t M, int64_t N,
                                int64_t K, const float* scale, const uint32_t* partial, int nparts,
                                float* scale_out, const Epilogue& ep, bool fast, hipStream_t stream) {
    const int64_t KT = (K + TILE_K - 1) / TILE_K;
    const unsigned grid = (unsigned)((M + TILE_N - 1) / TILE_N);
    const unsigned bt = 64 * SK_WAVES;
#define SK_LAUNCH(SRC)                                                                           \
    do {                                                                                         \
        if (fast)                                                                                \
            skinny_linear_kernel<SRC, true><<<grid, bt, 0, stream>>>(a, w, M, N, K, KT, scale,   \
                                                                     partial, nparts, scale_out, \
                                                                     ep);                        \
        else                                                                                     \
            skinny_linear_kernel<SRC, false><<<grid, bt, 0, stream>>>(a, w, M, N, K, KT, scale,  \
                                                                      partial, nparts,           \
                                                                      scale_out, ep);            \
    } while (0)
    if (adt == SRC_CODES) SK_LAUNCH(SRC_CODES);
    else if (adt == IN_BF16) SK_LAUNCH(IN_BF16);
    else SK_LAUNCH(IN_F16);
#undef SK_LAUNCH
    return hipGetLastError();
}

}  // namespace bql
