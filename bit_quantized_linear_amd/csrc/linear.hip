// Linear kernels for gfx950: the FP8 GEMM Y = (sA*sW[n])*(Aq.Wq^T) (vLLM
// PR #4118), the weight-only fp8 linear (optimum-quanto PR #241) and the
// W4A8 per-channel integer linear (QQQ issue #15).
//
// Two regimes, as the micro-benchmark on vLLM PR #4118 shows (small token
// counts are a weight-streaming problem, large ones a matrix-core problem):
//   * small M (<= 16 rows of A; W8A16 at every M): a streaming kernel.  Each
//     wave walks k-tiles of a block's 16-channel weight strip (two strips
//     per block when N is large), loading every MFMA operand straight from
//     HBM with unconditional 16-byte buffer loads (the packed layout makes
//     one wave-wide load 1 KiB contiguous; offsets past a descriptor's range
//     read zeros) into two register sets used in turn, so that the next
//     batch is in flight while one is multiplied.  A is read where it is: fp16
//     row-major (W8A16), 8-bit row-major (pre-quantized fp8 / int8), or
//     quantized by the kernel itself into LDS (fp8 with dynamic scaling,
//     M <= 4, or M <= 16 with M*K <= 16384).  Waves of a block split K and are summed through LDS in a
//     fixed order; blocks may split K further, with partials summed in a
//     fixed order by a second kernel.  Deterministic, no atomics.
//   * large M: block-tiled MFMA kernels.  Both operands live in HBM in the
//     MFMA operand tile layout (weights by prepack, 8-bit activations by
//     the quantizer or a repack), so each 1 KiB of a stage is one
//     buffer_load ... lds instruction that writes LDS directly (no VGPR
//     staging, no address scatter).  A ring of S stages keeps k-tiles in
//     flight; waits on the vector-memory counter are explicit because the
//     compiler does not track these LDS writes.  Output tiles are handed to
//     the 8 XCDs in contiguous ranges.  The epilogue converts and stages
//     each 16-row band through LDS and writes it with 16-byte stores.
//     Three main loops (plain, register-prefetching, k-split) are chosen
//     per shape by run_gemm.
#include <atomic>

#include "linear_common.h"

namespace bql {

// A operand of the small-M kernels, read through a buffer descriptor over
// one 16-row tile of A (rows past M lie outside it and read as zero; k past
// K or past the block's split of K gets an out-of-range offset and reads zero
// too).  The layout is fixed per call, so the lane's offsets are set
// up once as base + kt * per-k-tile stride + chunk stride and every load in
// the loop is an unconditional buffer load.
//   W8A16: row-major fp16; lane l takes row l%16, k0 .. k0+31 with
//          k0 = 128 kt + 32 (l/16), as four 16-byte loads.
//   8-bit row-major (small M): the lane's 32 bytes of the operand tile,
//          row l%16, k0 .. k0+31, as two 16-byte loads.
//   8-bit packed: the lane's two 16-byte chunks of the 2 KiB tile.
template <int V>
struct ALoader {
    static constexpr int CH = VT<V>::A_CHUNKS;
    static constexpr int KC = (V == V_W8A16 || V == V_W4A16G) ? 8 : 16;  // k per 16-byte chunk
    __amdgpu_buffer_rsrc_t rs;
    uint32_t base, skt, sc;  // lane's byte offset at kt = 0; strides per k-tile and per chunk
    int64_t kcol, klim;      // k of the lane's first element at kt = 0; chunks at k >= klim read zero
    __device__ ALoader(const LinParams& p, int64_t mt, int lane, int64_t kt_end) {
        const int64_t left = p.M - mt * 16;
        const int64_t rows = left < 16 ? left : 16;
        const int64_t r = lane & 15;
        kcol = 32 * (lane >> 4);
        klim = kt_end * TILE_K < p.K ? kt_end * TILE_K : p.K;
        const uint8_t* ptr;
        int64_t bytes;
        if (V == V_W8A16 || V == V_W4A16G) {
            ptr = (const uint8_t*)p.a + mt * 16 * p.K * 2;
            bytes = rows * p.K * 2;
            base = (uint32_t)((r * p.K + kcol) * 2);
            skt = TILE_K * 2;
            sc = 16;
        } else if (p.a_rowmajor) {
            ptr = (const uint8_t*)p.a + mt * 16 * p.K;
            bytes = rows * p.K;
            base = (uint32_t)(r * p.K + kcol);
            skt = TILE_K;
            sc = 16;
        } else {
            ptr = (const uint8_t*)p.a + mt * p.KT * 2048;
            bytes = p.KT * 2048;
            base = (uint32_t)(lane * 16);
            skt = 2048;
            sc = 1024;
        }
        rs = __builtin_amdgcn_make_buffer_rsrc((void*)ptr, (short)0, (int)bytes, 0x00020000);
    }
    __device__ __forceinline__ void load(u4 (&f)[CH], int64_t kt) const {
        constexpr uint32_t OOB = 0x7FFFFFF0u;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bool v = kcol + kt * TILE_K + KC * c < klim;
            const uint32_t off = base + (uint32_t)kt * skt + c * sc;
            f[c] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(v ? off : OOB), 0, 0));
        }
    }
};

// --------------------------------------------------------------- small M

// FUSED (fp8 variants, M <= 4, or M <= 16 with a short K): the kernel
// quantizes A itself.  Every block reads all of A for the per-tensor amax
// (a max, so every block gets the same scale bit for bit), then casts the A
// slice its K split needs into LDS as [M][slice] codes.  One launch instead
// of amax, cast and GEMV.
// With a static scale (p.given_scale) the amax is skipped.
// Fused blocks of two strips request both register sets' first batches
// before the prologue (measured 4 % faster at M = 1, N = 28672, K = 4096;
// with one strip per block it measured 1-11 % slower at N = 4096 and 6144).
constexpr bool gemv_early_batches(bool fused, int nt) { return fused && nt == 2; }

// Occupancy the small-M kernels are compiled for (waves per SIMD): enough
// register room for two weight batches, A and the decoded operands without
// spilling (both batches held through the fused prologue need 5), and as
// many resident blocks as that leaves.
constexpr int gemv_min_waves(int v, bool fused, int nt) {
    if (gemv_early_batches(fused, nt)) return 5;
    return (fused || v == V_FP8 || v == V_W4A8) ? 6 : 5;  // V_W8A16, V_W4A8G, V_W4A16G: 5
}

template <int V, int NT, int WAVES, int U, bool FUSED>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(gemv_min_waves(V, FUSED, NT), 8))) void gemv_kernel(LinParams p) {
    using Acc = typename VT<V>::Acc;
    constexpr int BT = VT<V>::B_TILE;
    extern __shared__ __attribute__((aligned(16))) uint8_t aq_lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t ntiles = p.N / TILE_N;
    const int64_t nt0 = (int64_t)blockIdx.x * NT;
    const int split = blockIdx.y;
    const int64_t mt = blockIdx.z;
    const int64_t kt_begin = split * p.kt_per_split;
    const int64_t kt_end = kt_begin + p.kt_per_split < p.KT ? kt_begin + p.kt_per_split : p.KT;
    const int g = lane >> 4;

    // Loads below are unconditional buffer loads: an offset past the
    // descriptor's range reads zeros without touching memory, so no load sits
    // in a branch and the compiler's waits count exactly the loads a value
    // needs (a branch around a load makes it wait for every load).
    constexpr uint32_t OOB = 0x7FFFFFF0u;
    const int64_t strips = ntiles - nt0 < NT ? ntiles - nt0 : NT;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w + nt0 * p.KT * BT), (short)0, (int)(strips * p.KT * BT), 0x00020000);
    // V_W4A8G, V_W4A16G: group scales [KT][N] fp32
    [[maybe_unused]] const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.ep.w_scale, (short)0, (int)((V == V_W4A8G || V == V_W4A16G) ? p.KT * p.N * 4 : 0),
        0x00020000);
    // Weight tiles for k-tiles kt, kt + WAVES, ... (U of them) of this wave;
    // tiles past this split's k range (or past N) read as zero.
    auto load_batch = [&](int64_t kt, u4 (&b)[U][NT][VT<V>::B_CHUNKS]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = kt + u * WAVES;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const bool ok = k < kt_end && j < strips;
                const uint32_t off = (uint32_t)((j * p.KT + k) * BT) + lane * 16;
                if constexpr (V == V_W4A8G || V == V_W4A16G) {
                    // the weight tile, then this k-tile's scale of the lane's channel
                    b[u][j][0] = __builtin_bit_cast(
                        u4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(ok ? off : OOB), 0, 2));
                    const uint32_t soff = (uint32_t)((k * p.N + (nt0 + j) * TILE_N + (lane & 15)) * 4);
                    b[u][j][1] = u4{(uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                                        rsc, (int)(ok ? soff : OOB), 0, 0),
                                    0u, 0u, 0u};
                } else {
#pragma unroll
                    for (int c = 0; c < VT<V>::B_CHUNKS; ++c)
                        b[u][j][c] = __builtin_bit_cast(
                            u4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(ok ? off + c * 1024 : OOB), 0, 2));
                }
            }
        }
    };
    // FUSED with one K split (the block's slice is all of A): the first
    // HOLD*T vectors of A are loaded once, before the weights, and kept for
    // the cast. Loads retire in issue order, so A issued first arrives
    // without waiting for the weight tiles behind it. (With several splits
    // the held vectors still feed the amax; the cast reloads its slice.)
    constexpr int T = 64 * WAVES, HOLD = FUSED ? 4 : 1;
    const bool whole = FUSED && p.splits == 1;
    const int64_t nvec = p.M * p.K / 8;  // K is a multiple of 16
    u4 held[HOLD];
    if constexpr (FUSED) {
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            (void*)p.a, (short)0, (int)(nvec * 16), 0x00020000);
#pragma unroll
        for (int h = 0; h < HOLD; ++h) {
            const int64_t i = threadIdx.x + (int64_t)h * T;
            held[h] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 ra, (int)(i < nvec ? i * 16 : OOB), 0, 0));
        }
    }
    // The first batch of weights is requested next, so its HBM latency
    // overlaps the scale computation and the A cast below (with early
    // batches, the second register set's batch too).
    constexpr bool EARLY = gemv_early_batches(FUSED, NT);
    u4 bq[U][NT][VT<V>::B_CHUNKS];
    u4 bo[U][NT][VT<V>::B_CHUNKS];
    load_batch(kt_begin + wave, bq);
    if constexpr (EARLY) load_batch(kt_begin + wave + WAVES * U, bo);

    float sa = 1.0f;
    if constexpr (FUSED) {
        __shared__ uint32_t sh[16];
        const uint16_t* x = (const uint16_t*)p.a;
        uint32_t mb = 0;
        const bool given = p.given_scale != nullptr;  // uniform: a static scale, no amax
        auto fold = [&](const u4& v) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = mag16(v[j] & 0xFFFFu), hi = mag16(v[j] >> 16);
                mb = mb > lo ? mb : lo;
                mb = mb > hi ? mb : hi;
            }
        };
        if (given) {
            sa = *p.given_scale;
        } else {
#pragma unroll
            for (int h = 0; h < HOLD; ++h) fold(held[h]);
            for (int64_t i = threadIdx.x + (int64_t)HOLD * T; i < nvec; i += T) fold(((const u4*)x)[i]);
            mb = block_max_u32(mb, sh);
            const float amax = p.xdt == IN_BF16 ? to_f32<IN_BF16>(mb) : to_f32<IN_F16>(mb);
            sa = amax == 0.0f ? 1.0f : amax / 448.0f;  // IEEE division, as the standalone quantizer
            if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) {
                if (p.scale_out) *p.scale_out = sa;
                if (p.scale_ws) *p.scale_ws = sa;
            }
        }
        // x / sA as the standalone quantizer forms it: from the reciprocal
        // with one residual correction where that is the IEEE quotient's code
        // for every input (the scale's range check), else the IEEE division.
        // enc2(a, b) gives the code pair of a / sA and b / sA; the input type
        // is a template argument (DT), so each value converts in one step.
        auto codes8 = [&](const u4& v, auto enc2, auto dt) {
            constexpr int DT = decltype(dt)::value;
            uint32_t c[4];  // code pairs
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = enc2(to_f32<DT>(v[j] & 0xFFFFu), to_f32<DT>(v[j] >> 16));
            return u2{c[0] | (c[1] << 16), c[2] | (c[3] << 16)};
        };
        // A is small here (at most 16 rows of a short K), so 32-bit indices
        const uint32_t slice = (uint32_t)(p.kt_per_split * TILE_K), k_lo = (uint32_t)(kt_begin * TILE_K);
        const uint32_t nv = (uint32_t)nvec, kk_ = (uint32_t)p.K, mm = (uint32_t)p.M;
        auto cast_dt = [&](auto enc2, auto dt) {
            auto codes = [&](const u4& v) { return codes8(v, enc2, dt); };
            if (whole) {
                // slice = [0, KT*128): cast the K real columns, zero the padding
                const uint32_t vpr = kk_ / 8;  // vectors per row
#pragma unroll
                for (int h = 0; h < HOLD; ++h) {
                    const uint32_t i = threadIdx.x + (uint32_t)h * T;
                    if (i < nv) *(u2*)(aq_lds + (i / vpr) * slice + (i % vpr) * 8) = codes(held[h]);
                }
                for (uint32_t i = threadIdx.x + (uint32_t)HOLD * T; i < nv; i += T)
                    *(u2*)(aq_lds + (i / vpr) * slice + (i % vpr) * 8) = codes(((const u4*)x)[i]);
                const uint32_t pad = (slice - kk_) / 8;  // zero 8-byte items past K in each row
                for (uint32_t i = threadIdx.x; i < mm * pad; i += T)
                    *(u2*)(aq_lds + (i / pad) * slice + kk_ + (i % pad) * 8) = u2{0, 0};
            } else {
                const uint32_t items = mm * slice / 8;
                for (uint32_t i = threadIdx.x; i < items; i += T) {
                    const uint32_t m = i / (slice / 8), kk = (i % (slice / 8)) * 8, k = k_lo + kk;
                    const u2 c = k < kk_ ? codes(*(const u4*)(x + (size_t)m * kk_ + k)) : u2{0, 0};
                    *(u2*)(aq_lds + m * slice + kk) = c;
                }
            }
        };
        auto cast_all = [&](auto enc2) {
            if (p.xdt == IN_BF16) cast_dt(enc2, DtTag<IN_BF16>{});
            else cast_dt(enc2, DtTag<IN_F16>{});
        };
        if (given) {
            const double inv = 1.0 / (double)sa;
            cast_all([&](float a, float b) { return e4m3_encode2(quot_f32(a, inv), quot_f32(b, inv)); });
        } else {
            const float y = 1.0f / sa;
            if (recip_div_ok(sa))
                cast_all([&](float a, float b) { return e4m3_div2_finite(a, b, sa, y); });
            else
                cast_all([&](float a, float b) { return e4m3_encode2(a / sa, b / sa); });
        }
        __syncthreads();
    } else if constexpr (V == V_FP8 || V == V_FP8X) {
        sa = *p.ep.a_scale;
    }

    Acc acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = Acc{0, 0, 0, 0};
    const ALoader<V> aload(p, mt, lane, kt_end);

    // Register double buffering: the next batch is in flight while this one
    // is multiplied, with the two register sets used in turn (a copy of the
    // next batch into the current one would wait for it to arrive). Loads
    // retire in issue order, so the A loads of a batch are issued before the
    // next batch of weights: the multiply waits for A and its own batch only.
    // Every load is unconditional (tiles past this split's range read as zero
    // without touching memory): a branch around a load makes the compiler
    // wait for all outstanding loads at the join.
    auto load_a = [&](int64_t kt, u4 (&a)[U][VT<V>::A_CHUNKS]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = kt + u * WAVES;
            if constexpr (FUSED) {
                // rows past M and k-tiles past the split read a valid LDS
                // address and are then replaced by zero
                const int row = lane & 15;
                const bool ok = k < kt_end && row < p.M;
                const uint8_t* t = aq_lds + (ok ? row * p.kt_per_split * TILE_K + (k - kt_begin) * TILE_K + 32 * g : 0);
                const u4 x0 = *(const u4*)t, x1 = *(const u4*)(t + 16);
                a[u][0] = ok ? x0 : u4{0, 0, 0, 0};
                a[u][1] = ok ? x1 : u4{0, 0, 0, 0};
            } else {
                aload.load(a[u], k);
            }
        }
    };
    auto multiply = [&](const u4 (&a)[U][VT<V>::A_CHUNKS], const u4 (&cur)[U][NT][VT<V>::B_CHUNKS]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NT; ++j) mma<V>(acc[j], a[u], cur[u][j]);
    };
    auto step = [&](int64_t kt, const u4 (&cur)[U][NT][VT<V>::B_CHUNKS], u4 (&nxt)[U][NT][VT<V>::B_CHUNKS]) {
        u4 a[U][VT<V>::A_CHUNKS];
        load_a(kt, a);
        load_batch(kt + WAVES * U, nxt);
        // keep the loads above the multiplies (the scheduler would sink them)
        __builtin_amdgcn_sched_barrier(0);
        multiply(a, cur);
    };
    // Two steps per trip; the second may lie past the split's range, where
    // both operands read as zero.  With early batches the first trip's
    // first step has its batch already requested and loads nothing.
    int64_t kt0 = kt_begin + wave;
    if constexpr (EARLY) {
        if (kt0 < kt_end) {
            u4 a[U][VT<V>::A_CHUNKS];
            load_a(kt0, a);
            multiply(a, bq);
            step(kt0 + WAVES * U, bo, bq);
        }
        kt0 += 2 * WAVES * U;
    }
    for (int64_t kt = kt0; kt < kt_end; kt += 2 * WAVES * U) {
        step(kt, bq, bo);
        step(kt + WAVES * U, bo, bq);
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

// Fixed-order sum of the split-K partials, then the epilogue: four
// consecutive outputs of a row per thread (N is a multiple of 16), read
// with 16-byte loads from each split and written with one store.  The
// partials are dead after this read: nontemporal loads keep them from
// displacing cached data (measured 1.4 % faster on the fp8 step at M = 1024).
template <int V>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(LinParams p) {
    using E = typename VT<V>::E;
    using E4 = E __attribute__((ext_vector_type(4)));
    const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4, total = p.M * p.N;
    if (idx >= total) return;
    const E* part = (const E*)p.partial;
    E4 s = __builtin_nontemporal_load((const E4*)(part + idx));
    for (int k = 1; k < p.splits; ++k) s += __builtin_nontemporal_load((const E4*)(part + k * total + idx));
    const float sa = (V == V_FP8 || V == V_FP8X) ? *p.ep.a_scale : 1.0f;
    const int64_t m = idx / p.N, n = idx % p.N;
    uint32_t b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) b[t] = out_bits<V>(p.ep, sa, m, n + t, s[t]);
    uint8_t* y = (uint8_t*)p.ep.y;
    const int esz = out_size(p.ep.ydt);
    const int64_t at = (m * p.ep.ldy + n) * esz;
    if (esz == 4) *(u4*)(y + at) = u4{b[0], b[1], b[2], b[3]};
    else if (esz == 2) *(u2*)(y + at) = u2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
    else *(uint32_t*)(y + at) = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
}

template <int V>
static hipError_t launch_splitk_reduce(const LinParams& p, hipStream_t stream) {
    const int64_t quads = p.M * p.N / 4;
    splitk_reduce_kernel<V><<<(unsigned)((quads + 255) / 256), 256, 0, stream>>>(p);
    return hipGetLastError();
}

// --------------------------------------------------------------- large M

// The A operand of the k-split tile kernel: a block's BM rows of A, either packed
// into 16x128 operand tiles (2 KiB each, [16-row strip][k-tile]) or
// row-major [M,K] bytes (E4M3 codes or int8) where the caller keeps them.
// Both give the same LDS image: the 16-byte load of (strip s, half h) by
// lane l holds row 16 s + l % 16 and k = 128 kt + 32 (l / 16) + 16 h ..
// +15 of the block's rows (the packed layout stores exactly that there).
// Rows past M lie past the descriptor's range and chunks past K (a multiple
// of 16) get an offset past it, so both read as zero.
struct ATiles {
    __amdgpu_buffer_rsrc_t rsrc;
    int KT;
    int K;
    bool rowmajor;
};

template <int BM>
__device__ __forceinline__ ATiles a_tiles(const LinParams& p, int64_t m0) {
    ATiles t;
    t.KT = (int)p.KT;
    t.K = (int)p.K;
    t.rowmajor = p.a_rowmajor != 0;
    if (t.rowmajor) {
        const int64_t rows = p.M - m0 < BM ? p.M - m0 : BM;  // <= 256 rows of K <= 2^22 bytes
        t.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)p.a + m0 * p.K), (short)0,
                                                   (int)(rows * p.K), 0x00020000);
    } else {
        const int64_t mt0 = m0 / 16, mtiles = (p.M + 15) / 16;
        const int64_t strips = mtiles - mt0 < BM / 16 ? mtiles - mt0 : BM / 16;
        t.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)p.a + mt0 * p.KT * 2048),
                                                   (short)0, (int)(strips * p.KT * 2048), 0x00020000);
    }
    return t;
}

__device__ __forceinline__ int a_tile_offset(const ATiles& t, int strip, int h, int kt, int lane) {
    if (t.rowmajor) {
        const int k = kt * 128 + 32 * (lane >> 4) + 16 * h;
        return k < t.K ? (strip * 16 + (lane & 15)) * t.K + k : 0x7FFFFFF0;
    }
    return (strip * t.KT + kt) * 2048 + h * 1024 + lane * 16;
}

// One 16 x 16 accumulator tile's raw sums (fp32, or the int32 of the W4A8
// kernels) into split blockIdx.y's partial buffer [M][N]; rows past M and
// columns past N are skipped.
template <int V>
__device__ __forceinline__ void store_partial_tile(const LinParams& p, const typename VT<V>::Acc& a,
                                                   int64_t r0, int64_t c0, int lane) {
    using E = typename VT<V>::E;
    E* part = (E*)p.partial + (int64_t)blockIdx.y * p.M * p.N;
    const int64_t n = c0 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t m = r0 + 4 * (lane >> 4) + r;
        if (m < p.M && n < p.N) part[m * p.N + n] = a[r];
    }
}

template <int V, int FM, int FN>
__device__ __forceinline__ void store_partials(const LinParams& p, const typename VT<V>::Acc (&acc)[FM][FN],
                                               int64_t r0, int64_t c0, int lane) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) store_partial_tile<V>(p, acc[i][j], r0 + i * 16, c0 + j * 16, lane);
}

template <int V, int BM, int BN, int WM, int WN, int S>
struct GemmCfg {
    static constexpr int NW = WM * WN;
    static constexpr int BT = VT<V>::B_TILE;
    static constexpr int A_BYTES = (BM / 16) * 2048;
    static constexpr int B_BYTES = (BN / 16) * BT;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = S * STAGE;
    static constexpr int FM = BM / (16 * WM), FN = BN / (16 * WN);
    static constexpr int A_LD = A_BYTES / 1024, B_LD = B_BYTES / 1024;  // 1 KiB loads per stage
    static constexpr int LDPW = (A_LD + B_LD) / NW;
    static_assert(A_LD % NW == 0 && B_LD % NW == 0, "stage loads must split evenly over waves");
    static_assert(LDPW * (S - 1) < 64, "vmcnt range");
    // epilogue scratch: one 16-row band of a wave's tile, 4 bytes per value, padded rows
    static constexpr int EPI_ROW = FN * 16 * 4 + 16;
    static constexpr int EPI_WAVE = 16 * EPI_ROW;
    static_assert(EPI_WAVE * NW <= LDS, "epilogue scratch must fit in the stage buffers");
};

template <int V, int BM, int BN, int WM, int WN, int S>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(LinParams p) {
    using C = GemmCfg<V, BM, BN, WM, WN, S>;
    using Acc = typename VT<V>::Acc;
    constexpr int NW = C::NW, FM = C::FM, FN = C::FN, BT = C::BT;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int64_t bm, bn;
    tile_coords(blockIdx.x, (p.M + BM - 1) / BM, (p.N + BN - 1) / BN, bm, bn);
    const int64_t m0 = bm * BM, n0 = bn * BN;
    const int64_t mt0 = m0 / 16, nt0 = n0 / 16;
    const int64_t mtiles = (p.M + 15) / 16, ntiles = p.N / 16;
    const int KT = (int)p.KT;

    // Buffer descriptors over this block's own strips; loads past them
    // (rows beyond M, channels beyond N) return zeros.
    const int64_t a_strips = mtiles - mt0 < BM / 16 ? mtiles - mt0 : BM / 16;
    const int64_t b_strips = ntiles - nt0 < BN / 16 ? ntiles - nt0 : BN / 16;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)p.a + mt0 * p.KT * 2048), (short)0, (int)(a_strips * p.KT * 2048),
        0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w + nt0 * p.KT * BT), (short)0, (int)(b_strips * p.KT * BT), 0x00020000);

    auto issue = [&](int kt, int stage) {
        uint8_t* base = lds + stage * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::A_LD / NW; ++i) {
            const int slot = wave + NW * i, sub = slot >> 1, h = slot & 1;
            const int off = (sub * KT + kt) * 2048 + h * 1024 + lane * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(base + slot * 1024), 16, off, 0,
                                                     0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::B_LD / NW; ++i) {
            const int slot = wave + NW * i;
            int off;
            if constexpr (BT == 2048) off = ((slot >> 1) * KT + kt) * 2048 + (slot & 1) * 1024 + lane * 16;
            else off = (slot * KT + kt) * 1024 + lane * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(base + C::A_BYTES + slot * 1024),
                                                     16, off, 0, 0, 0);
        }
    };

    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Acc{0, 0, 0, 0};

#pragma unroll
    for (int s = 0; s < S - 1; ++s)
        if (s < KT) issue(s, s);

    for (int kt = 0; kt < KT; ++kt) {
        // This wave's loads of stage kt are done once no more than the loads
        // of the stages issued after it are outstanding.
        const int after = (KT - 1 - kt) < (S - 2) ? (KT - 1 - kt) : (S - 2);
        if (after == S - 2) wait_vmcnt<C::LDPW * (S - 2)>();
        else if (S > 3 && after == 1) wait_vmcnt<C::LDPW>();
        else if (S > 4 && after == 2) wait_vmcnt<C::LDPW * 2>();
        else wait_vmcnt<0>();
        // every wave's share of stage kt is in LDS, and every wave has
        // finished reading the stage that the next issue overwrites
        lds_barrier();
        if (kt + S - 1 < KT) issue(kt + S - 1, (kt + S - 1) % S);

        const uint8_t* base = lds + (kt % S) * C::STAGE;
        const uint8_t* abase = base + (wm * FM) * 2048 + lane * 16;
        const uint8_t* bbase = base + C::A_BYTES + (wn * FN) * BT + lane * 16;
        if constexpr (V == V_FP8) {
            v8i bf[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = as_v8i(*(const u4*)(bbase + j * BT), *(const u4*)(bbase + j * BT + 1024));
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const v8i af =
                    as_v8i(*(const u4*)(abase + i * 2048), *(const u4*)(abase + i * 2048 + 1024));
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma_fp8(af, bf[j], acc[i][j]);
            }
        } else if constexpr (V == V_FP8X) {
            v8h bh[FN][4];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                decode32(*(const u4*)(bbase + j * BT), *(const u4*)(bbase + j * BT + 1024), bh[j]);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                v8h ah[4];
                decode32(*(const u4*)(abase + i * 2048), *(const u4*)(abase + i * 2048 + 1024), ah);
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[i][j] = mfma_f16(ah[q], bh[j][q], acc[i][j]);
            }
        } else {  // V_W4A8
            u4 bf[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) bf[j] = *(const u4*)(bbase + j * BT);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const u4 alo = *(const u4*)(abase + i * 2048);
                const u4 ahi = *(const u4*)(abase + i * 2048 + 1024);
#pragma unroll
                for (int j = 0; j < FN; ++j) mma_w4a8(acc[i][j], alo, ahi, bf[j]);
            }
        }
    }

    // ---- epilogue: per wave, per 16-row band: convert, stage in LDS, 16-byte stores
    __syncthreads();  // all waves are done with the stage buffers
    const float sa = (V == V_FP8 || V == V_FP8X) ? *p.ep.a_scale : 1.0f;
    const int esz = out_size(p.ep.ydt);
    uint8_t* scratch = lds + wave * C::EPI_WAVE;
    const int chunks_per_row = FN * 16 * esz / 16;
    const int64_t col0 = n0 + wn * FN * 16;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t rbase = m0 + (wm * FM + i) * 16;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int c = j * 16 + (lane & 15);
            const int64_t n = col0 + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * (lane >> 4) + r;
                const uint32_t bits = (n < p.N && rbase + row < p.M)
                                          ? out_bits<V>(p.ep, sa, rbase + row, n, acc[i][j][r])
                                          : 0u;
                uint8_t* d = scratch + row * C::EPI_ROW + c * esz;
                if (esz == 4) *(uint32_t*)d = bits;
                else if (esz == 2) *(uint16_t*)d = (uint16_t)bits;
                else *d = (uint8_t)bits;
            }
        }
        // the band is written and read back by this wave only
        __builtin_amdgcn_wave_barrier();
        for (int q = lane; q < 16 * chunks_per_row; q += 64) {
            const int row = q / chunks_per_row, ch = q % chunks_per_row;
            const int64_t m = rbase + row;
            const int64_t n = col0 + (int64_t)ch * 16 / esz;
            if (m < p.M && n < p.N)
                *(u4*)((uint8_t*)p.ep.y + (m * p.ep.ldy + n) * esz) =
                    *(const u4*)(scratch + row * C::EPI_ROW + ch * 16);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Same tiling, with the fragments of k-tile kt+1 read from LDS into a
// second register set while the MFMAs of k-tile kt run. Every wave holds
// k-tile kt in registers before the barrier of iteration kt, so that
// iteration refills slot kt % S with k-tile kt + S: S = 2 already keeps one
// k-tile of DMA in flight behind the one being read.
// Per-group W4A8 runs four waves of 64x64 outputs each (fewer LDS bytes per
// MFMA than eight waves of 64x32); capped at 256 registers so that two
// waves share a SIMD (two blocks per CU) without spilling.
template <int V, int BM, int BN, int WM, int WN, int S>
__global__ __launch_bounds__(64 * WM * WN)
__attribute__((amdgpu_waves_per_eu(V == V_W4A8G ? 2 : 1, 8))) void gemm_pipe_kernel(LinParams p) {
    using C = GemmCfg<V, BM, BN, WM, WN, S>;
    using Acc = typename VT<V>::Acc;
    constexpr int NW = C::NW, FM = C::FM, FN = C::FN, BT = C::BT;
    constexpr int BC = VT<V>::B_CHUNKS;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int64_t bm, bn;
    tile_coords(blockIdx.x, (p.M + BM - 1) / BM, (p.N + BN - 1) / BN, bm, bn);
    const int64_t m0 = bm * BM, n0 = bn * BN;
    const int64_t mt0 = m0 / 16, nt0 = n0 / 16;
    const int64_t mtiles = (p.M + 15) / 16, ntiles = p.N / 16;
    // k-tiles kt0 .. kt0 + KT - 1 (split blockIdx.y of K); KS strides strips
    const int KS = (int)p.KT, kt0 = (int)(blockIdx.y * p.kt_per_split);
    const int KT = (int)(p.KT - kt0 < p.kt_per_split ? p.KT - kt0 : p.kt_per_split);

    const int64_t a_strips = mtiles - mt0 < BM / 16 ? mtiles - mt0 : BM / 16;
    const int64_t b_strips = ntiles - nt0 < BN / 16 ? ntiles - nt0 : BN / 16;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)p.a + mt0 * p.KT * 2048), (short)0, (int)(a_strips * p.KT * 2048),
        0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w + nt0 * p.KT * BT), (short)0, (int)(b_strips * p.KT * BT), 0x00020000);

    auto issue = [&](int kt, int stage) {
        uint8_t* base = lds + stage * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::A_LD / NW; ++i) {
            const int slot = wave + NW * i, sub = slot >> 1, h = slot & 1;
            const int off = (sub * KS + kt0 + kt) * 2048 + h * 1024 + lane * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(base + slot * 1024), 16, off, 0,
                                                     0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::B_LD / NW; ++i) {
            const int slot = wave + NW * i;
            int off;
            if constexpr (BT == 2048) off = ((slot >> 1) * KS + kt0 + kt) * 2048 + (slot & 1) * 1024 + lane * 16;
            else off = (slot * KS + kt0 + kt) * 1024 + lane * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(base + C::A_BYTES + slot * 1024),
                                                     16, off, 0, 0, 0);
        }
    };
    // Wait until this wave's loads of a k-tile are complete, given how many
    // k-tiles it has issued after that one (at most S - 1).
    auto wait_behind = [&](int after) {
        if (S > 1 && after >= S - 1) wait_vmcnt<C::LDPW * (S - 1)>();
        else if (S > 2 && after == S - 2) wait_vmcnt<C::LDPW * (S - 2)>();
        else if (S > 3 && after == 1) wait_vmcnt<C::LDPW>();
        else wait_vmcnt<0>();
    };
    struct Frag {
        u4 a[FM][2];
        u4 b[FN][BC];
    };
    auto read_frags = [&](int kt, Frag& f) {
        const uint8_t* base = lds + (kt % S) * C::STAGE;
        const uint8_t* abase = base + (wm * FM) * 2048 + lane * 16;
        const uint8_t* bbase = base + C::A_BYTES + (wn * FN) * BT + lane * 16;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int c = 0; c < BC; ++c) f.b[j][c] = *(const u4*)(bbase + j * BT + c * 1024);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            f.a[i][0] = *(const u4*)(abase + i * 2048);
            f.a[i][1] = *(const u4*)(abase + i * 2048 + 1024);
        }
    };

    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Acc{0, 0, 0, 0};

    // V_W4A8G: the block's group scales / 16, [KT][BN] fp32 after the stage ring
    [[maybe_unused]] const float* gsc = (const float*)(lds + C::LDS);
    auto compute = [&](const Frag& f, [[maybe_unused]] int kt) {
        if constexpr (V == V_FP8) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const v8i af = as_v8i(f.a[i][0], f.a[i][1]);
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma_fp8(af, as_v8i(f.b[j][0], f.b[j][1]), acc[i][j]);
            }
        } else if constexpr (V == V_FP8X) {
            v8h bh[FN][4];
#pragma unroll
            for (int j = 0; j < FN; ++j) decode32(f.b[j][0], f.b[j][1], bh[j]);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                v8h ah[4];
                decode32(f.a[i][0], f.a[i][1], ah);
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[i][j] = mfma_f16(ah[q], bh[j][q], acc[i][j]);
            }
        } else if constexpr (V == V_W4A8G) {
            float sc[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) sc[j] = gsc[kt * BN + (wn * FN + j) * 16 + (lane & 15)];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) group_fold(acc[i][j], f.a[i][0], f.a[i][1], f.b[j][0], sc[j]);
        } else {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) mma_w4a8(acc[i][j], f.a[i][0], f.a[i][1], f.b[j][0]);
        }
    };

#pragma unroll
    for (int s = 0; s < S; ++s)
        if (s < KT) issue(s, s);
    if constexpr (V == V_W4A8G) {
        // stage the block's group scales (columns past N read as zero); the
        // barrier's wait also retires the first stages' DMA, which the loop
        // below would wait for next anyway
        float* g = (float*)(lds + C::LDS);
        for (int q = tid; q < KT * BN; q += 64 * NW) {
            const int64_t n = n0 + q % BN;
            g[q] = n < p.N ? p.ep.w_scale[(int64_t)(kt0 + q / BN) * p.N + n] * 0.0625f : 0.0f;  // scale / 16
        }
        __syncthreads();
    }
    // One k-step with a successor (kt + 1 < KT): fragments of kt are in
    // `cur`, those of kt+1 are read into `nxt` while the MFMAs of kt run.
    // The body has no branch around the LDS reads, so the MFMAs only wait
    // for `cur`, whose reads completed before the barrier.
    auto step = [&](int kt, Frag& cur, Frag& nxt) {
        // k-tiles kt+2 .. min(kt+S-1, KT-1) were issued after kt+1
        wait_behind(KT - 2 - kt < S - 2 ? KT - 2 - kt : S - 2);
        lds_barrier();
        if (kt + S < KT) issue(kt + S, kt % S);
        read_frags(kt + 1, nxt);
        compute(cur, kt);
    };
    Frag f0, f1;
    wait_behind(KT - 1 < S - 1 ? KT - 1 : S - 1);
    lds_barrier();
    read_frags(0, f0);
    // unrolled by two so that the two fragment sets swap roles without copies
    int kt = 0;
    for (; kt + 2 < KT; kt += 2) {
        step(kt, f0, f1);
        step(kt + 1, f1, f0);
    }
    if (kt + 1 < KT) {
        step(kt, f0, f1);
        compute(f1, kt + 1);
    } else {
        compute(f0, kt);
    }

    // ---- epilogue (as gemm_kernel); with K split over blocks, this split's
    // raw sums go to its partial buffer for the split-K reduce
    __syncthreads();
    wait_vmcnt<0>();
    if (p.splits > 1) {
        store_partials<V, FM, FN>(p, acc, m0 + wm * FM * 16, n0 + wn * FN * 16, lane);
        return;
    }
    const float sa = (V == V_FP8 || V == V_FP8X) ? *p.ep.a_scale : 1.0f;
    const int esz = out_size(p.ep.ydt);
    uint8_t* scratch = lds + wave * C::EPI_WAVE;
    const int chunks_per_row = FN * 16 * esz / 16;
    const int64_t col0 = n0 + wn * FN * 16;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t rbase = m0 + (wm * FM + i) * 16;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int c = j * 16 + (lane & 15);
            const int64_t n = col0 + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * (lane >> 4) + r;
                const uint32_t bits = (n < p.N && rbase + row < p.M)
                                          ? out_bits<V>(p.ep, sa, rbase + row, n, acc[i][j][r])
                                          : 0u;
                uint8_t* d = scratch + row * C::EPI_ROW + c * esz;
                if (esz == 4) *(uint32_t*)d = bits;
                else if (esz == 2) *(uint16_t*)d = (uint16_t)bits;
                else *d = (uint8_t)bits;
            }
        }
        __builtin_amdgcn_wave_barrier();
        for (int q = lane; q < 16 * chunks_per_row; q += 64) {
            const int row = q / chunks_per_row, ch = q % chunks_per_row;
            const int64_t m = rbase + row;
            const int64_t n = col0 + (int64_t)ch * 16 / esz;
            if (m < p.M && n < p.N)
                *(u4*)((uint8_t*)p.ep.y + (m * p.ep.ldy + n) * esz) =
                    *(const u4*)(scratch + row * C::EPI_ROW + ch * 16);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Exact fp8 tile kernel with the k range split between two groups of
// waves. Every 16x128 operand tile holds, per lane, two 16-byte halves that
// feed two f16 MFMAs each; wave group g reads and decodes only half g of
// each tile, so a wave with a 64x64 output tile decodes two fp8 pairs per
// MFMA instead of four and reads half the LDS bytes. The two groups' fp32
// partial sums are added through LDS at the end (each group finishes half of
// the rows; a + b == b + a, so the result does not depend on which group).
template <int BM, int BN, int WM, int WN, int S>
struct KsCfg {
    static constexpr int SW = WM * WN, NW = 2 * SW;
    static constexpr int A_BYTES = (BM / 16) * 2048, B_BYTES = (BN / 16) * 2048;
    static constexpr int STAGE = A_BYTES + B_BYTES, RING = S * STAGE;
    static constexpr int FM = BM / (16 * WM), FN = BN / (16 * WN);
    static constexpr int A_LD = A_BYTES / 1024, B_LD = B_BYTES / 1024;
    static constexpr int LDPW = (A_LD + B_LD) / NW;
    static constexpr int XCH = (FM / 2) * FN * 4 * 64 * 4;  // bytes a wave hands to its partner
    static constexpr int EPI_ROW = FN * 16 * 4 + 16, EPI_WAVE = 16 * EPI_ROW;
    static constexpr int LDS0 = RING > NW * XCH ? RING : NW * XCH;
    static constexpr int LDS = LDS0 > NW * EPI_WAVE ? LDS0 : NW * EPI_WAVE;
    static_assert(A_LD % NW == 0 && B_LD % NW == 0, "stage loads must split evenly over waves");
    static_assert(FM % 2 == 0, "each group finishes half of a wave's row tiles");
    static_assert(LDPW * (S - 1) < 64, "vmcnt range");
};

template <int BM, int BN, int WM, int WN, int S>
__global__ __launch_bounds__(128 * WM * WN) void gemm_ks_kernel(LinParams p) {
    using C = KsCfg<BM, BN, WM, WN, S>;
    constexpr int NW = C::NW, SW = C::SW, FM = C::FM, FN = C::FN;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = wave / SW, sw = wave % SW, wm = sw / WN, wn = sw % WN;
    int64_t bm, bn;
    tile_coords(blockIdx.x, (p.M + BM - 1) / BM, (p.N + BN - 1) / BN, bm, bn);
    const int64_t m0 = bm * BM, n0 = bn * BN;
    const int64_t nt0 = n0 / 16, ntiles = p.N / 16;
    // k-tiles kt0 .. kt0 + KT - 1 (split blockIdx.y of K); KS strides strips
    const int KS = (int)p.KT, kt0 = (int)(blockIdx.y * p.kt_per_split);
    const int KT = (int)(p.KT - kt0 < p.kt_per_split ? p.KT - kt0 : p.kt_per_split);

    // A packed or row-major (see ATiles)
    const int64_t b_strips = ntiles - nt0 < BN / 16 ? ntiles - nt0 : BN / 16;
    const ATiles at = a_tiles<BM>(p, m0);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w + nt0 * p.KT * 2048), (short)0, (int)(b_strips * p.KT * 2048), 0x00020000);

    auto issue = [&](int kt, int stage) {
        uint8_t* base = lds + stage * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::A_LD / NW; ++i) {
            const int slot = wave + NW * i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(at.rsrc, (lds_ptr_t)(base + slot * 1024), 16,
                                                     a_tile_offset(at, slot >> 1, slot & 1, kt0 + kt, lane),
                                                     0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::B_LD / NW; ++i) {
            const int slot = wave + NW * i;
            const int off = ((slot >> 1) * KS + kt0 + kt) * 2048 + (slot & 1) * 1024 + lane * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(base + C::A_BYTES + slot * 1024),
                                                     16, off, 0, 0, 0);
        }
    };
    auto wait_behind = [&](int after) {
        if (S > 1 && after >= S - 1) wait_vmcnt<C::LDPW * (S - 1)>();
        else if (S > 2 && after == S - 2) wait_vmcnt<C::LDPW * (S - 2)>();
        else if (S > 3 && after == 1) wait_vmcnt<C::LDPW>();
        else wait_vmcnt<0>();
    };
    struct Frag {
        u4 a[FM];
        u4 b[FN];
    };
    auto read_frags = [&](int kt, Frag& f) {
        const uint8_t* base = lds + (kt % S) * C::STAGE + g * 1024 + lane * 16;
#pragma unroll
        for (int j = 0; j < FN; ++j) f.b[j] = *(const u4*)(base + C::A_BYTES + (wn * FN + j) * 2048);
#pragma unroll
        for (int i = 0; i < FM; ++i) f.a[i] = *(const u4*)(base + (wm * FM + i) * 2048);
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0, 0, 0, 0};

    auto compute = [&](const Frag& f) {
        v8h bh[FN][2];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            bh[j][0] = e4m3x8_to_f16(f.b[j][0], f.b[j][1]);
            bh[j][1] = e4m3x8_to_f16(f.b[j][2], f.b[j][3]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const v8h a0 = e4m3x8_to_f16(f.a[i][0], f.a[i][1]);
            const v8h a1 = e4m3x8_to_f16(f.a[i][2], f.a[i][3]);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                acc[i][j] = mfma_f16(a0, bh[j][0], acc[i][j]);
                acc[i][j] = mfma_f16(a1, bh[j][1], acc[i][j]);
            }
        }
    };
    auto step = [&](int kt, Frag& cur, Frag& nxt) {
        wait_behind(KT - 2 - kt < S - 2 ? KT - 2 - kt : S - 2);
        lds_barrier();
        if (kt + S < KT) issue(kt + S, kt % S);
        read_frags(kt + 1, nxt);
        compute(cur);
    };

#pragma unroll
    for (int s = 0; s < S; ++s)
        if (s < KT) issue(s, s);
    Frag f0, f1;
    wait_behind(KT - 1 < S - 1 ? KT - 1 : S - 1);
    lds_barrier();
    read_frags(0, f0);
    int kt = 0;
    for (; kt + 2 < KT; kt += 2) {
        step(kt, f0, f1);
        step(kt + 1, f1, f0);
    }
    if (kt + 1 < KT) {
        step(kt, f0, f1);
        compute(f1);
    } else {
        compute(f0);
    }

    // ---- add the two groups' partial sums: group 0 finishes row tiles
    // [0, FM/2) of its wave tile, group 1 row tiles [FM/2, FM)
    wait_vmcnt<0>();
    __syncthreads();
    const bool low = g == 0;
    {
        float* out = (float*)(lds + wave * C::XCH);
#pragma unroll
        for (int i = 0; i < FM; ++i)
            if ((i < FM / 2) != low)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        out[(((i % (FM / 2)) * FN + j) * 4 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    {
        const float* in = (const float*)(lds + ((1 - g) * SW + sw) * C::XCH);
#pragma unroll
        for (int i = 0; i < FM; ++i)
            if ((i < FM / 2) == low)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[i][j][r] += in[(((i % (FM / 2)) * FN + j) * 4 + r) * 64 + lane];
    }
    __syncthreads();

    // with K split over blocks, this split's raw sums (each group's half of
    // the row tiles) go to its partial buffer for the split-K reduce
    if (p.splits > 1) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            if ((i < FM / 2) != low) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j)
                store_partial_tile<V_FP8X>(p, acc[i][j], m0 + (wm * FM + i) * 16, n0 + (wn * FN + j) * 16, lane);
        }
        return;
    }

    // ---- epilogue: per 16-row band, values staged in LDS, 16-byte stores
    const float sa = *p.ep.a_scale;
    const int esz = out_size(p.ep.ydt);
    uint8_t* scratch = lds + wave * C::EPI_WAVE;
    const int chunks_per_row = FN * 16 * esz / 16;
    const int64_t col0 = n0 + wn * FN * 16;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        if ((i < FM / 2) != low) continue;
        const int64_t rbase = m0 + (wm * FM + i) * 16;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int c = j * 16 + (lane & 15);
            const int64_t n = col0 + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * (lane >> 4) + r;
                const uint32_t bits = (n < p.N && rbase + row < p.M)
                                          ? out_bits<V_FP8X>(p.ep, sa, rbase + row, n, acc[i][j][r])
                                          : 0u;
                uint8_t* d = scratch + row * C::EPI_ROW + c * esz;
                if (esz == 4) *(uint32_t*)d = bits;
                else if (esz == 2) *(uint16_t*)d = (uint16_t)bits;
                else *d = (uint8_t)bits;
            }
        }
        __builtin_amdgcn_wave_barrier();
        for (int q = lane; q < 16 * chunks_per_row; q += 64) {
            const int row = q / chunks_per_row, ch = q % chunks_per_row;
            const int64_t m = rbase + row;
            const int64_t n = col0 + (int64_t)ch * 16 / esz;
            if (m < p.M && n < p.N)
                *(u4*)((uint8_t*)p.ep.y + (m * p.ep.ldy + n) * esz) =
                    *(const u4*)(scratch + row * C::EPI_ROW + ch * 16);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// ------------------------------------------------------------------ host

constexpr int GEMV_U = 2;       // weight k-tiles per wave per batch
constexpr int GEMV_WAVES = 8;   // measured faster than 16 at every M = 1 Llama shape
constexpr int MAX_SPLITS = 8;
constexpr int SMALL_M = (int)SMALL_M_MAX;
constexpr int FUSED_M = 16;                // small-M fp8 calls that quantize A in-kernel
constexpr int64_t FUSED_LDS = 48 * 1024;   // bytes of A codes a fused block may stage

bool use_small_m(int variant, int64_t M, int64_t N, int64_t K) {
    if (variant == V_W4A16G) return M <= SMALL_M || !w4a16_tile_fits(M, N, K);
    return variant == V_W8A16 || M <= SMALL_M;
}

struct GemvPlan {
    int64_t KT, kt_per_split;
    int splits;
};

// Blocks of GEMV_WAVES waves stream one 16-channel strip each.  Few strips
// (short N) leave CUs idle, so K may be split across blocks (with a
// fixed-order reduce): up to about 256 blocks, or 512 when K is short
// (KT < 32), keeping at least 8 (4) k-tiles per split.  Of those split
// counts the plan takes the cheapest by a cost fitted to timings of M <= 16
// fp8 linears on MI355X with N = 1024-2048: a block streams its strip's
// weight bytes at about 45 GB/s after a fixed start (A comes from L2), and
// a K split adds the reduce launch and the partial sums, about 3.6 us.
// Short strips are therefore not split (M = 1, N = K = 2048: 9.3 -> 5.5 us;
// M = 16, N = 1024, K = 8192: 15.5 -> 14.2 us), long ones are (M = 1,
// N = 1024, K = 16384: four splits, 9.8 us against 10.5 unsplit).
static GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int variant) {
    GemvPlan pl;
    pl.KT = (K + TILE_K - 1) / TILE_K;
    const int64_t groups = (N / TILE_N) * ((M + 15) / 16);
    const int64_t target = pl.KT < 32 ? 512 : 256, min_kt = pl.KT < 32 ? 4 : 8;
    int smax = 1;
    if (M <= SMALL_M)
        while (groups * smax < target && smax * 2 <= MAX_SPLITS && pl.KT / (smax * 2) >= min_kt)
            smax *= 2;
    const bool int4 = variant == V_W4A8 || variant == V_W4A8G || variant == V_W4A16G;
    const double strip_bytes = (double)pl.KT * (int4 ? INT4_TILE_BYTES : 2048);
    constexpr double BLOCK_BYTES_PER_US = 45e3, SPLIT_US = 3.6;
    int s = 1;
    double best = strip_bytes / BLOCK_BYTES_PER_US;
    for (int c = 2; c <= smax; c *= 2) {
        const double cost = SPLIT_US + strip_bytes / c / BLOCK_BYTES_PER_US;
        if (cost < best) {
            best = cost;
            s = c;
        }
    }
    pl.kt_per_split = (pl.KT + s - 1) / s;
    pl.splits = (int)((pl.KT + pl.kt_per_split - 1) / pl.kt_per_split);
    return pl;
}

size_t w4a16_ws_bytes(int64_t M, int64_t N, int64_t K) {
    if (use_small_m(V_W4A16G, M, N, K)) return small_m_ws_bytes(M, N, K, V_W4A16G);
    const int s = w4a16_tile_splits(M, N, K);
    const int64_t KT = K / TILE_K, per = (KT + s - 1) / s, splits = (KT + per - 1) / per;
    return splits > 1 ? (size_t)splits * M * N * 4 : 0;
}

size_t small_m_ws_bytes(int64_t M, int64_t N, int64_t K, int variant) {
    if (!use_small_m(variant, M, N, K) || M > SMALL_M) return 0;
    GemvPlan pl = plan_gemv(M, N, K, variant);
    return pl.splits > 1 ? (size_t)pl.splits * M * N * 4 : 0;
}

// Every fused block reads all of A for the amax and casts its slice, so
// above M = 4 fusing pays only while A is small: measured 29 % faster at
// M = 16, K = 1024 (two launches fewer), 45 % slower at M = 16, K = 4096.
bool fused_small_m(int64_t M, int64_t N, int64_t K) {
    if (M > FUSED_M || (M > 4 && M * K > 16384)) return false;
    GemvPlan pl = plan_gemv(M, N, K, V_FP8X);
    return M * pl.kt_per_split * TILE_K <= FUSED_LDS;
}

template <int V, bool FUSED>
static hipError_t run_gemv(LinParams p, hipStream_t stream) {
    const int64_t strips = p.N / TILE_N;
    const size_t lds = FUSED ? (size_t)(p.M * p.kt_per_split * TILE_K) : 0;
    // With many strips (fp8, N >= 16384) a block takes two strips at one
    // k-tile per wave per batch (the same registers): half as many blocks
    // to start, reduce and retire, measured 4-5 % faster at N = 28672.
    // Fewer strips keep one per block, so that every CU gets a block.
    if constexpr (V == V_FP8 || V == V_FP8X) {
        if (strips >= 1024 && p.splits == 1) {
            dim3 grid((unsigned)((strips + 1) / 2), 1, (unsigned)((p.M + 15) / 16));
            gemv_kernel<V, 2, GEMV_WAVES, 1, FUSED><<<grid, 64 * GEMV_WAVES, lds, stream>>>(p);
            return hipGetLastError();
        }
    }
    dim3 grid((unsigned)strips, (unsigned)p.splits, (unsigned)((p.M + 15) / 16));
    gemv_kernel<V, 1, GEMV_WAVES, GEMV_U, FUSED><<<grid, 64 * GEMV_WAVES, lds, stream>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_reduce<V>(p, stream);
}

template <int V, int BM, int BN, int WM, int WN, int S>
static hipError_t launch_gemm(const LinParams& p, hipStream_t stream) {
    using C = GemmCfg<V, BM, BN, WM, WN, S>;
    // Dynamic LDS above 64 KiB needs the attribute, set once per device
    // (before any graph capture can happen: the first launch is eager).
    static std::atomic<uint64_t> configured{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = uint64_t(1) << (dev & 63);
    if (!(configured.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute((const void*)gemm_kernel<V, BM, BN, WM, WN, S>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
        if (e != hipSuccess) return e;
        configured.fetch_or(bit, std::memory_order_acq_rel);
    }
    const int64_t blocks = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    gemm_kernel<V, BM, BN, WM, WN, S><<<(unsigned)blocks, 64 * WM * WN, C::LDS, stream>>>(p);
    return hipGetLastError();
}

template <int V, int BM, int BN, int WM, int WN, int S>
static hipError_t launch_gemm_pipe(const LinParams& p, hipStream_t stream) {
    using C = GemmCfg<V, BM, BN, WM, WN, S>;
    // V_W4A8G stages its group scales ([KT][BN] fp32) after the stage ring
    constexpr int MAX_LDS = V == V_W4A8G ? C::LDS + BN * W4A8G_MAX_KT * 4 : C::LDS;
    const int lds = V == V_W4A8G ? C::LDS + BN * (int)p.KT * 4 : C::LDS;
    static std::atomic<uint64_t> configured{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = uint64_t(1) << (dev & 63);
    if (!(configured.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute((const void*)gemm_pipe_kernel<V, BM, BN, WM, WN, S>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, MAX_LDS);
        if (e != hipSuccess) return e;
        configured.fetch_or(bit, std::memory_order_acq_rel);
    }
    const int64_t blocks = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    gemm_pipe_kernel<V, BM, BN, WM, WN, S><<<dim3((unsigned)blocks, (unsigned)p.splits), 64 * WM * WN, lds,
                                             stream>>>(p);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int S>
static hipError_t launch_gemm_ks(const LinParams& p, hipStream_t stream) {
    using C = KsCfg<BM, BN, WM, WN, S>;
    static std::atomic<uint64_t> configured{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = uint64_t(1) << (dev & 63);
    if (!(configured.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute((const void*)gemm_ks_kernel<BM, BN, WM, WN, S>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
        if (e != hipSuccess) return e;
        configured.fetch_or(bit, std::memory_order_acq_rel);
    }
    const int64_t blocks = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    gemm_ks_kernel<BM, BN, WM, WN, S><<<dim3((unsigned)blocks, (unsigned)p.splits), 128 * WM * WN, C::LDS,
                                        stream>>>(p);
    return hipGetLastError();
}



// Kernel choice for the tiled path, from measured M=1024 sweeps on the
// Llama-3-8B projection shapes (fp8) and K = N in 4096..8192 (W4A8). "One tile per CU" shapes (at most 256
// 128x128 tiles) favour kernels that hide latency inside one block: the
// k-split exact kernel and the register-prefetching fp8 kernel with a
// three-stage ring; shapes with many 256x256 tiles favour the big fp8 tile.
constexpr int64_t CUS = 256;
// Exact fp8 runs the 256-row kernel of gemm_exact.hip where exact_plan
// takes the shape (M > 128); below that, with at most one 128x128 output
// tile per CU, the k-split kernel.
static bool uses_ks(int variant, int64_t M, int64_t N, int64_t K) {
    return variant == V_FP8X && exact_plan(M, N, K).fn == 0 && ((M + 127) / 128) * ((N + 127) / 128) <= CUS;
}

// Row-major 8-bit A (per-lane gathers of 16-byte chunks from 16 rows)
// costs the tile kernels that re-read A from L2 for many column tiles more
// than a repack launch: at M = 1024, +3 % for the exact 128x128 kernel at
// N = 28672 and +37 % for W4A8, against -5 to -9 % for the k-split kernel.
bool reads_rowmajor_a(int variant, int64_t M, int64_t N, int64_t K) {
    return use_small_m(variant, M, N, K) || uses_ks(variant, M, N, K);
}

// K splits of the 128 x 128 tile kernels that take them (the exact k-split
// kernel, the register-prefetch kernel: fast fp8 with at most one tile per
// CU, W4A8 per channel and per group).  With few output tiles most CUs idle
// while each block walks all of K (M = 128 and 256 at these N), so K is split
// over blocks whose raw sums go to fp32 / int32 partials and the split-K
// reduce.  Cost in k-tile times of one block: ceil(blocks / CUs) rounds of
// ceil(KT / s) k-tiles, plus the partials' write and read (8 bytes per
// output and split; a 128 x 128 block's k-tile takes about as long as the
// chip moves 4 MB).  At most 8 splits of 4+ k-tiles.
static bool tile_splittable(int variant, int64_t M, int64_t N, int64_t K) {
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    if (variant == V_FP8X) return uses_ks(variant, M, N, K);
    if (variant == V_FP8) return t128 <= CUS;
    return variant == V_W4A8 || variant == V_W4A8G;
}

static int tile_splits(int variant, int64_t M, int64_t N, int64_t K) {
    if (use_small_m(variant, M, N, K)) return 1;
    if (variant == V_FP8X && exact_plan(M, N, K).fn != 0) return exact_plan(M, N, K).splits;
    if (!tile_splittable(variant, M, N, K)) return 1;
    constexpr double BYTES_PER_KTILE = 4e6;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128), kt = (K + TILE_K - 1) / TILE_K;
    int best = 1;
    double best_cost = (double)((tiles + CUS - 1) / CUS) * kt;
    for (int sp = 2; sp <= MAX_SPLITS && kt / sp >= 4; ++sp) {
        const double cost = (double)((tiles * sp + CUS - 1) / CUS) * ((kt + sp - 1) / sp) +
                            (double)sp * M * N * 8 / BYTES_PER_KTILE;
        if (cost < best_cost) {
            best = sp;
            best_cost = cost;
        }
    }
    return best;
}

size_t split_ws_bytes(int64_t M, int64_t N, int64_t K, int variant) {
    if (variant == V_W4A16G) return w4a16_ws_bytes(M, N, K);
    if (use_small_m(variant, M, N, K)) return small_m_ws_bytes(M, N, K, variant);
    const int sp = tile_splits(variant, M, N, K);
    const int64_t kt = (K + TILE_K - 1) / TILE_K, per = (kt + sp - 1) / sp, n = (kt + per - 1) / per;
    return n > 1 ? (size_t)n * M * N * 4 : 0;
}

template <int V>
static hipError_t run_gemm_kernel(const LinParams& p, hipStream_t stream);

// The tile kernel chosen by run_gemm_kernel, with K split over blocks when
// tile_splits says so (then the split-K reduce applies the epilogue).
template <int V>
static hipError_t run_gemm(const LinParams& p0, hipStream_t stream) {
    LinParams p = p0;
    const int sp = tile_splits(V, p.M, p.N, p.K);
    if (sp > 1) {
        p.kt_per_split = (p.KT + sp - 1) / sp;
        p.splits = (int)((p.KT + p.kt_per_split - 1) / p.kt_per_split);
    }
    hipError_t e = run_gemm_kernel<V>(p, stream);
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_reduce<V>(p, stream);
}

template <int V>
static hipError_t run_gemm_kernel(const LinParams& p, hipStream_t stream) {
    const int64_t t128 = ((p.M + 127) / 128) * ((p.N + 127) / 128);
    const int64_t t256 = ((p.M + 255) / 256) * ((p.N + 255) / 256);
    if constexpr (V == V_FP8X) {
        // M > 128: the 256-row kernel (at least four times the MFMAs per
        // A conversion of the 64x64-per-wave kernels), with its K splits
        const ExactPlan xp = exact_plan(p.M, p.N, p.K);
        if (xp.fn != 0) return launch_gemm_exact(p, xp, stream);
        // at most one 128x128 tile per CU: a four-stage ring, so that each
        // k-tile's DMA has three k-tiles of compute to land behind
        if (uses_ks(V, p.M, p.N, p.K)) return launch_gemm_ks<128, 128, 2, 2, 4>(p, stream);
        // Two blocks share a CU, so the busiest CU carries ceil(tiles / CUs)
        // tiles: 128x96 tiles win where they even that out (M = 1024, N =
        // 6144: 384 tiles of 128 columns leave half the CUs with two, 512
        // tiles of 96 give every CU two of three quarters the width).
        const int64_t t96 = ((p.M + 127) / 128) * ((p.N + 95) / 96);
        if (((t96 + CUS - 1) / CUS) * 96 < ((t128 + CUS - 1) / CUS) * 128)
            return launch_gemm<V, 128, 96, 2, 2, 2>(p, stream);
        return launch_gemm<V, 128, 128, 2, 2, 2>(p, stream);
    } else if constexpr (V == V_FP8) {
        if (t128 <= CUS) return launch_gemm_pipe<V, 128, 128, 4, 2, 4>(p, stream);
        if (t256 >= 3 * CUS / 2) return launch_gemm<V, 256, 256, 4, 4, 2>(p, stream);
        return launch_gemm<V, 128, 128, 2, 4, 2>(p, stream);
    } else if constexpr (V == V_W4A8G) {  // best at every K = N in 4096..8192 measured
        // at most one tile per CU (a block per CU at a time): a four-stage ring
        if (t128 * p.splits <= CUS) return launch_gemm_pipe<V, 128, 128, 2, 2, 4>(p, stream);
        return launch_gemm_pipe<V, 128, 128, 2, 2, 2>(p, stream);
    } else {  // per-channel W4A8: best at every K = N in 4096..8192 measured
        if (t128 * p.splits <= CUS) return launch_gemm_pipe<V, 128, 128, 2, 4, 4>(p, stream);
        return launch_gemm_pipe<V, 128, 128, 2, 4, 2>(p, stream);
    }
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
    p.xdt = args.xdt;
    p.scale_out = args.scale_out;
    p.scale_ws = args.scale_ws;
    p.a_rowmajor = args.a_rowmajor;
    p.given_scale = args.given_scale;
    if (use_small_m(args.variant, args.M, args.N, args.K)) {
        GemvPlan pl = plan_gemv(args.M, args.N, args.K, args.variant);
        p.KT = pl.KT;
        p.kt_per_split = pl.kt_per_split;
        p.splits = pl.splits;
        if (args.fused) {
            // read by the split-K reduce
            p.ep.a_scale = args.given_scale ? args.given_scale : args.scale_ws;
            if (args.variant == V_FP8) return run_gemv<V_FP8, true>(p, stream);
            return run_gemv<V_FP8X, true>(p, stream);
        }
        switch (args.variant) {
            case V_FP8: return run_gemv<V_FP8, false>(p, stream);
            case V_FP8X: return run_gemv<V_FP8X, false>(p, stream);
            case V_W8A16: return run_gemv<V_W8A16, false>(p, stream);
            case V_W4A8G: return run_gemv<V_W4A8G, false>(p, stream);
            case V_W4A16G: return run_gemv<V_W4A16G, false>(p, stream);
            default: return run_gemv<V_W4A8, false>(p, stream);
        }
    }
    if (args.variant == V_W4A16G) {
        p.KT = (args.K + TILE_K - 1) / TILE_K;
        const int s = w4a16_tile_splits(args.M, args.N, args.K);
        p.kt_per_split = (p.KT + s - 1) / s;
        p.splits = (int)((p.KT + p.kt_per_split - 1) / p.kt_per_split);
        hipError_t e = launch_gemm_w4a16(p, stream);
        if (e != hipSuccess || p.splits == 1) return e;
        return launch_splitk_reduce<V_W4A16G>(p, stream);
    }
    if (args.a_rowmajor && !reads_rowmajor_a(args.variant, args.M, args.N, args.K))
        return hipErrorInvalidValue;  // this shape's tile kernel takes packed A
    p.KT = (args.K + TILE_K - 1) / TILE_K;
    p.kt_per_split = p.KT;
    p.splits = 1;
    if (args.variant == V_FP8) return run_gemm<V_FP8>(p, stream);
    if (args.variant == V_FP8X) return run_gemm<V_FP8X>(p, stream);
    if (args.variant == V_W4A8G) return run_gemm<V_W4A8G>(p, stream);
    return run_gemm<V_W4A8>(p, stream);
}

}  // namespace bql
