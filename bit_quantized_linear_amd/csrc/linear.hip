// Linear kernels for gfx950: the FP8 GEMM Y = (sA*sW[n])*(Aq.Wq^T) (vLLM
// PR #4118), the weight-only fp8 linear (optimum-quanto PR #241) and the
// W4A8 per-channel integer linear (QQQ issue #15).
//
// Two regimes, as the micro-benchmark on vLLM PR #4118 shows (small token
// counts are a weight-streaming problem, large ones a matrix-core problem):
//   * small M (<= 16 rows of A): a streaming kernel.  Each wave walks k-tiles
//     of one or more 16-channel weight strips, loading every MFMA operand
//     straight from HBM with 16-byte loads (the packed layout makes one
//     wave-wide load 1 KiB contiguous), A rows padded to 16 by zero lanes.
//     Waves of a block split K and are summed through LDS in a fixed order;
//     blocks may split K further, with partials summed in a fixed order by
//     a second kernel.  Deterministic, no atomics.
//   * large M: a block-tiled MFMA kernel with both operands staged through
//     LDS in operand order, double buffered, fused scale epilogue.
#include "device.h"
#include "kernels.h"

namespace bql {

struct LinParams {
    const void* a;
    const uint8_t* w;
    int64_t M, N, K, KT;
    int64_t kt_per_split;
    int splits;
    void* partial;
    Epilogue ep;
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

// One lane's A operand for one k-tile: row `row`, k0 .. k0+31 (k0 = 128 kt
// + 32 g for lane group g), zero where the row or k does not exist.
template <int V>
__device__ __forceinline__ void load_a(u4 (&f)[VT<V>::A_CHUNKS], const void* A, int64_t row,
                                       bool ok, int64_t K, int64_t k0) {
    if constexpr (V == V_W8A16) {
        const uint16_t* p = (const uint16_t*)A + row * K + k0;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            f[c] = (ok && k0 + 8 * c < K) ? *(const u4*)(p + 8 * c) : u4{0, 0, 0, 0};
    } else {
        const uint8_t* p = (const uint8_t*)A + row * K + k0;
#pragma unroll
        for (int c = 0; c < 2; ++c)
            f[c] = (ok && k0 + 16 * c < K) ? *(const u4*)(p + 16 * c) : u4{0, 0, 0, 0};
    }
}

template <int V>
__device__ __forceinline__ void load_b(u4 (&f)[VT<V>::B_CHUNKS], const uint8_t* tile, int lane,
                                       bool ok) {
#pragma unroll
    for (int c = 0; c < VT<V>::B_CHUNKS; ++c)
        f[c] = ok ? __builtin_nontemporal_load((const u4*)(tile + c * 1024 + lane * 16))
                  : u4{0, 0, 0, 0};
}

template <int V>
__device__ __forceinline__ void mma(typename VT<V>::Acc& acc, const u4 (&a)[VT<V>::A_CHUNKS],
                                    const u4 (&b)[VT<V>::B_CHUNKS]) {
    if constexpr (V == V_FP8) {
        v8i av = {(int)a[0][0], (int)a[0][1], (int)a[0][2], (int)a[0][3],
                  (int)a[1][0], (int)a[1][1], (int)a[1][2], (int)a[1][3]};
        v8i bv = {(int)b[0][0], (int)b[0][1], (int)b[0][2], (int)b[0][3],
                  (int)b[1][0], (int)b[1][1], (int)b[1][2], (int)b[1][3]};
        acc = mfma_fp8(av, bv, acc);
    } else if constexpr (V == V_W4A8) {
        v4i alo = {(int)a[0][0], (int)a[0][1], (int)a[0][2], (int)a[0][3]};
        v4i ahi = {(int)a[1][0], (int)a[1][1], (int)a[1][2], (int)a[1][3]};
        v4i blo = {(int)int4_lo_x16(b[0][0]), (int)int4_lo_x16(b[0][1]),
                   (int)int4_lo_x16(b[0][2]), (int)int4_lo_x16(b[0][3])};
        v4i bhi = {(int)int4_hi_x16(b[0][0]), (int)int4_hi_x16(b[0][1]),
                   (int)int4_hi_x16(b[0][2]), (int)int4_hi_x16(b[0][3])};
        acc = mfma_i8(alo, blo, acc);
        acc = mfma_i8(ahi, bhi, acc);
    } else if constexpr (V == V_FP8X) {
        // four f16 MFMAs over k0+8q .. k0+8q+7 on losslessly decoded codes
        const uint32_t da[8] = {a[0][0], a[0][1], a[0][2], a[0][3], a[1][0], a[1][1], a[1][2], a[1][3]};
        const uint32_t db[8] = {b[0][0], b[0][1], b[0][2], b[0][3], b[1][0], b[1][1], b[1][2], b[1][3]};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            acc = mfma_f16(e4m3x8_to_f16(da[2 * q], da[2 * q + 1]),
                           e4m3x8_to_f16(db[2 * q], db[2 * q + 1]), acc);
    } else {  // W8A16: four f16 MFMAs over k0+8q .. k0+8q+7
        const uint32_t db[8] = {b[0][0], b[0][1], b[0][2], b[0][3], b[1][0], b[1][1], b[1][2], b[1][3]};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            acc = mfma_f16(__builtin_bit_cast(v8h, a[q]), e4m3x8_to_f16(db[2 * q], db[2 * q + 1]), acc);
    }
}

template <int V>
__device__ __forceinline__ void finish(const LinParams& p, float sa, int64_t m, int64_t n,
                                       typename VT<V>::E v) {
    if constexpr (V == V_W4A8) epilogue_int(p.ep, m, n, v);
    else epilogue_float(p.ep, sa, m, n, v);
}

// --------------------------------------------------------------- small M

template <int V, int NT, int WAVES, int U>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(LinParams p) {
    using Acc = typename VT<V>::Acc;
    constexpr int BT = VT<V>::B_TILE;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t ntiles = p.N / TILE_N;
    const int64_t nt0 = (int64_t)blockIdx.x * NT;
    const int split = blockIdx.y;
    const int64_t mt = blockIdx.z;
    const int64_t kt_begin = split * p.kt_per_split;
    const int64_t kt_end = kt_begin + p.kt_per_split < p.KT ? kt_begin + p.kt_per_split : p.KT;
    const int64_t row = mt * 16 + (lane & 15);
    const bool row_ok = row < p.M;
    const int g = lane >> 4;

    Acc acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = Acc{0, 0, 0, 0};

    for (int64_t kt = kt_begin + wave; kt < kt_end; kt += WAVES * U) {
        u4 a[U][VT<V>::A_CHUNKS];
        u4 b[U][NT][VT<V>::B_CHUNKS];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = kt + u * WAVES;
            const bool kv = k < kt_end;
            load_a<V>(a[u], p.a, row, row_ok && kv, p.K, k * TILE_K + 32 * g);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                load_b<V>(b[u][j], p.w + ((nt0 + j) * p.KT + k) * BT, lane,
                          kv && (nt0 + j) < ntiles);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NT; ++j) mma<V>(acc[j], a[u], b[u][j]);
    }

    if constexpr (WAVES > 1) {
        __shared__ Acc red[WAVES][NT][64];
#pragma unroll
        for (int j = 0; j < NT; ++j) red[wave][j][lane] = acc[j];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            Acc s = red[0][j][lane];
            for (int w = 1; w < WAVES; ++w) s += red[w][j][lane];
            acc[j] = s;
        }
    }

    const float sa = (V == V_FP8 || V == V_FP8X) ? *p.ep.a_scale : 1.0f;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        if (nt0 + j >= ntiles) continue;
        const int64_t n = (nt0 + j) * TILE_N + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = mt * 16 + 4 * g + i;
            if (m >= p.M) continue;
            if (p.splits == 1) {
                finish<V>(p, sa, m, n, acc[j][i]);
            } else {
                using E = typename VT<V>::E;
                ((E*)p.partial)[((int64_t)split * p.M + m) * p.N + n] = acc[j][i];
            }
        }
    }
}

// Fixed-order sum of the split-K partials, then the epilogue.
template <int V>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(LinParams p) {
    using E = typename VT<V>::E;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= p.M * p.N) return;
    const E* part = (const E*)p.partial;
    E s = part[idx];
    for (int k = 1; k < p.splits; ++k) s += part[(int64_t)k * p.M * p.N + idx];
    const float sa = (V == V_FP8 || V == V_FP8X) ? *p.ep.a_scale : 1.0f;
    finish<V>(p, sa, idx / p.N, idx % p.N, s);
}

// --------------------------------------------------------------- large M

template <int V, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_kernel(LinParams p) {
    using Acc = typename VT<V>::Acc;
    constexpr int BT = VT<V>::B_TILE;
    constexpr int ASUB = BM / TILE_N, BSUB = BN / TILE_N;
    constexpr int A_BYTES = ASUB * 2048;  // 8-bit A: a 16 x 128 sub-tile is 2 KiB
    constexpr int B_BYTES = BSUB * BT;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int FM = BM / 32, FN = BN / 32;  // 2 x 2 waves, 16 x 16 fragments
    constexpr int A_PER_T = A_BYTES / 16 / 256, B_PER_T = B_BYTES / 16 / 256;
    static_assert(A_PER_T * 256 * 16 == A_BYTES && B_PER_T * 256 * 16 == B_BYTES, "tile split");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int64_t nt0 = n0 / TILE_N, ntiles = p.N / TILE_N;
    const uint8_t* A = (const uint8_t*)p.a;

    u4 ra[A_PER_T], rb[B_PER_T];
    auto gload = [&](int64_t kt) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int q = tid + 256 * i, r = q >> 3, c = q & 7;
            const int64_t gm = m0 + r, gk = kt * TILE_K + c * 16;
            ra[i] = (gm < p.M && gk < p.K) ? *(const u4*)(A + gm * p.K + gk) : u4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int q = tid + 256 * i, j = q / (BT / 16), w = q % (BT / 16);
            rb[i] = (nt0 + j < ntiles)
                        ? __builtin_nontemporal_load((const u4*)(p.w + ((nt0 + j) * p.KT + kt) * BT + w * 16))
                        : u4{0, 0, 0, 0};
        }
    };
    auto sstore = [&](int buf) {
        uint8_t* base = lds + buf * STAGE;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int q = tid + 256 * i, r = q >> 3, c = q & 7;
            const int off = (r >> 4) * 2048 + (c & 1) * 1024 + ((r & 15) + 16 * (c >> 1)) * 16;
            *(u4*)(base + off) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int q = tid + 256 * i;
            *(u4*)(base + A_BYTES + q * 16) = rb[i];
        }
    };

    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Acc{0, 0, 0, 0};

    gload(0);
    sstore(0);
    __syncthreads();
    for (int64_t kt = 0; kt < p.KT; ++kt) {
        const int cur = (int)(kt & 1);
        const bool more = kt + 1 < p.KT;
        if (more) gload(kt + 1);
        const uint8_t* base = lds + cur * STAGE;
        u4 af[FM][2];
        u4 bf[FN][VT<V>::B_CHUNKS];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const uint8_t* t = base + (wm * FM + i) * 2048 + lane * 16;
            af[i][0] = *(const u4*)t;
            af[i][1] = *(const u4*)(t + 1024);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const uint8_t* t = base + A_BYTES + (wn * FN + j) * BT + lane * 16;
#pragma unroll
            for (int c = 0; c < VT<V>::B_CHUNKS; ++c) bf[j][c] = *(const u4*)(t + c * 1024);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) mma<V>(acc[i][j], af[i], bf[j]);
        if (more) sstore(cur ^ 1);
        __syncthreads();
    }

    const float sa = (V == V_FP8 || V == V_FP8X) ? *p.ep.a_scale : 1.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t n = n0 + (wn * FN + j) * 16 + (lane & 15);
            if (n >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + (wm * FM + i) * 16 + 4 * (lane >> 4) + r;
                if (m < p.M) finish<V>(p, sa, m, n, acc[i][j][r]);
            }
        }
}

// ------------------------------------------------------------------ host

constexpr int GEMV_WAVES = 8;
constexpr int GEMV_U = 2;
constexpr int MAX_SPLITS = 8;
constexpr int SMALL_M = 16;

bool use_small_m(int variant, int64_t M, int64_t N, int64_t K) {
    (void)N; (void)K;
    return variant == V_W8A16 || M <= SMALL_M;
}

struct GemvPlan {
    int64_t KT, kt_per_split;
    int splits;
};

static GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K) {
    GemvPlan pl;
    pl.KT = (K + TILE_K - 1) / TILE_K;
    const int64_t groups = N / TILE_N;
    const int64_t mtiles = (M + 15) / 16;
    int s = 1;
    if (M <= SMALL_M)
        while (groups * mtiles * s < 1024 && s * 2 <= MAX_SPLITS && pl.KT / (s * 2) >= 2) s *= 2;
    pl.kt_per_split = (pl.KT + s - 1) / s;
    pl.splits = (int)((pl.KT + pl.kt_per_split - 1) / pl.kt_per_split);
    return pl;
}

size_t small_m_ws_bytes(int64_t M, int64_t N, int64_t K, int variant) {
    if (!use_small_m(variant, M, N, K) || M > SMALL_M) return 0;
    GemvPlan pl = plan_gemv(M, N, K);
    return pl.splits > 1 ? (size_t)pl.splits * M * N * 4 : 0;
}

template <int V>
static hipError_t run_gemv(LinParams p, hipStream_t stream) {
    dim3 grid((unsigned)(p.N / TILE_N), (unsigned)p.splits, (unsigned)((p.M + 15) / 16));
    gemv_kernel<V, 1, GEMV_WAVES, GEMV_U><<<grid, 64 * GEMV_WAVES, 0, stream>>>(p);
    if (p.splits > 1) {
        const int64_t total = p.M * p.N;
        splitk_reduce_kernel<V><<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(p);
    }
    return hipGetLastError();
}

template <int V>
static hipError_t run_gemm(LinParams p, hipStream_t stream) {
    constexpr int BM = 128, BN = 128;
    dim3 grid((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM));
    gemm_kernel<V, BM, BN><<<grid, 256, 0, stream>>>(p);
    return hipGetLastError();
}

hipError_t launch_linear(const LinearArgs& args, void* ws, size_t ws_bytes, hipStream_t stream) {
    (void)ws_bytes;
    LinParams p;
    p.a = args.a;
    p.w = args.w;
    p.M = args.M;
    p.N = args.N;
    p.K = args.K;
    p.ep.y = args.y;
    p.ep.ldy = args.N;
    p.ep.ydt = args.ydt;
    p.ep.a_scale = args.a_scale;
    p.ep.w_scale = args.w_scale;
    p.ep.w_per_channel = args.w_per_channel;
    p.ep.out_scale = args.out_scale;
    p.partial = ws;
    if (use_small_m(args.variant, args.M, args.N, args.K)) {
        GemvPlan pl = plan_gemv(args.M, args.N, args.K);
        p.KT = pl.KT;
        p.kt_per_split = pl.kt_per_split;
        p.splits = pl.splits;
        switch (args.variant) {
            case V_FP8: return run_gemv<V_FP8>(p, stream);
            case V_FP8X: return run_gemv<V_FP8X>(p, stream);
            case V_W8A16: return run_gemv<V_W8A16>(p, stream);
            default: return run_gemv<V_W4A8>(p, stream);
        }
    }
    p.KT = (args.K + TILE_K - 1) / TILE_K;
    p.kt_per_split = p.KT;
    p.splits = 1;
    if (args.variant == V_FP8) return run_gemm<V_FP8>(p, stream);
    if (args.variant == V_FP8X) return run_gemm<V_FP8X>(p, stream);
    return run_gemm<V_W4A8>(p, stream);
}

}  // namespace bql
