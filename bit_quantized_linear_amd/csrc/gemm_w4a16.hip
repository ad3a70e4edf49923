// Per-group weight-only int4 tile kernel for larger M (QQQ issue #15, the
// "awq-g128" / "marlin-g128" rows: fp16 activations, int4 weights with one
// fp16 scale per output channel and 128-k group):
//   Y[m,n] = sum_g s[n,g] * sum_{k in g} A[m,k] * W4[n,k]
// Each group's sum is formed on the f16 matrix cores (fp16 x small-integer
// products are exact, summed in fp32) and folded into the fp32 accumulator
// with one fused multiply-add by the group scale.
//
// Organisation (gfx950: 4 SIMDs per CU, 160 KiB LDS per CU):
//   * A block computes a 128 x 256 (or, where that fills the CUs better,
//     128 x 128) output tile with four waves side by side in N, one per SIMD;
//     each wave owns all 128 rows and 64 (32) channels: 32 (16) output tiles
//     of 16 x 16 whose fp32 accumulators stay in ordinary vector registers,
//     because the per-group fold is vector-ALU work.  The int4
//     decode (about 44 vector instructions per 16-channel x 128-k weight
//     tile) is paid once per 8 row strips, and the fold once per 4 MFMAs.
//   * A (row-major fp16 in HBM) reaches LDS by LDS-DMA (buffer_load ... lds),
//     one k-tile (128 rows x 256 bytes, 32 KiB) per stage, four stages in
//     the ring.  In LDS a row's sixteen 16-byte pieces are stored at slot
//     piece ^ (row % 16): the DMA still reads 256 contiguous bytes per row,
//     and the operand reads (lane l: row l % 16, piece 4 (l / 16) + c) touch
//     16 distinct slots per 16 lanes, so they are free of bank conflicts.
//   * The packed int4 tiles (1 KiB per 16 channels x 128 k, the layout of
//     the prepacked weight) and the group scales are loaded straight into
//     registers one k-tile ahead: each wave reads only its own channels.
//   * Loop order inside a k-tile: channel strip j outer, row strip i inner,
//     so that each decoded weight tile is held once (two buffers: the next
//     one decodes while the current one multiplies) and the eight A operand
//     strips stay in registers for the whole k-tile; in the last strip pass
//     every A strip is replaced by the next k-tile's right after its last use.
//   * Output tiles go to the 8 XCDs in contiguous ranges; the epilogue stages
//     the wave's 128-row tile in LDS and writes it with 16-byte stores.
#include <atomic>
#include <type_traits>

#include "linear_common.h"

namespace bql {

namespace {

constexpr int QM = 128;                    // block rows
constexpr int QW = 4;                      // waves per block, side by side in N
constexpr int QFM = QM / 16;               // 16-row strips per wave (8)
constexpr int QSTAGE = QM * 256;           // one k-tile of A: 32 KiB
constexpr int QS = 4;                      // LDS ring depth
constexpr int QLDS = QS * QSTAGE;          // 128 KiB
constexpr int QLD = QFM;                   // A DMA instructions per wave per stage

// Block geometry for QFN 16-channel strips per wave (4: 128 x 256 blocks,
// 2: 128 x 128).
template <int QFN>
struct QCfg {
    static constexpr int QN = QW * QFN * 16;              // block columns
    static constexpr int EPI_ROW = QFN * 16 * 4 + 16;     // staged row: up to 16 QFN fp32, padded
    static constexpr int EPI_WAVE = QM * EPI_ROW;
    static constexpr int LDS_ALL = QLDS > QW * EPI_WAVE ? QLDS : QW * EPI_WAVE;
    static_assert(LDS_ALL <= 160 * 1024, "LDS");
    static_assert(QLD + 2 * QFN < 64, "vmcnt range");
};

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Writes the wave's staged 128 x 16 QFN tile (OUT bits, EPI_ROW bytes per
// row) to y (row stride ldy elements) with 16-byte stores.  N is a multiple
// of 16, so a store's columns lie all inside or all outside N.
template <int OUT, int QFN>
__device__ __forceinline__ void copy_out(const LinParams& p, uint8_t* y, int64_t ldy, const uint8_t* band,
                                         int64_t m0, int64_t col0, int lane) {
    constexpr int ESZ = OUT == OUT_F32 ? 4 : 2, QEPI_ROW = QCfg<QFN>::EPI_ROW;
    constexpr int CHUNKS = QFN * 16 * ESZ / 16, ITERS = QM * CHUNKS / 64;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int q = lane + 64 * it, row = q / CHUNKS, ch = q % CHUNKS;
        const int64_t m = m0 + row, n = col0 + ch * (16 / ESZ);
        const u4 v = *(const u4*)(band + row * QEPI_ROW + ch * 16);
        if (m < p.M && n < p.N) *(u4*)(y + (m * ldy + n) * ESZ) = v;
    }
}

// Part h (0..7) of the decode of a lane's 16 packed int4 bytes into eight
// fp16-pair words: dword h / 2, its low nibbles (even h: k0 + 4 (h/2) ..)
// or its high nibbles (odd h: k0 + 16 + 4 (h/2) ..), as words 2 (h/2),
// 2 (h/2) + 1 (+ 8 for the high nibbles) of e.  Eight parts spread the
// decode over the steps of a strip pass.
__device__ __forceinline__ void dec_part(const u4& src, int h, uint32_t (&e)[16]) {
    const int q = h >> 1;
    if (h & 1) int4x4_to_f16(src[q] >> 4, e[8 + 2 * q], e[8 + 2 * q + 1]);
    else int4x4_to_f16(src[q], e[2 * q], e[2 * q + 1]);
}

__device__ __forceinline__ v8h as_op(const uint32_t (&e)[16], int q) {
    return __builtin_bit_cast(v8h, v4i{(int)e[4 * q], (int)e[4 * q + 1], (int)e[4 * q + 2], (int)e[4 * q + 3]});
}

// Instruction order of one step (a row strip of a strip pass), for the
// scheduler: each of its 4 MFMAs followed by two vector instructions (the
// previous group sum's fold and a part of the next weight decode), then the
// rest, then in the last pass the step's 4 operand reads of the next k-tile.
// Nothing moves across steps.
__device__ __forceinline__ void step_order(bool reads) {
    constexpr int MFMA = 0x008, VALU = 0x002, DS_READ = 0x100;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(VALU, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(VALU, 8, 0);
    if (reads) __builtin_amdgcn_sched_group_barrier(DS_READ, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace

template <int QFN>
__global__ __launch_bounds__(64 * QW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_w4a16_kernel(LinParams p) {
    constexpr int QN = QCfg<QFN>::QN, QEPI_ROW = QCfg<QFN>::EPI_ROW, QEPI_WAVE = QCfg<QFN>::EPI_WAVE;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // the wave index and the tile coordinates (whose 64-bit divisions run on
    // the vector ALU) are uniform: read them as such, so that the buffer
    // descriptors built from them stay scalar
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int64_t bm, bn;
    tile_coords(blockIdx.x, (p.M + QM - 1) / QM, (p.N + QN - 1) / QN, bm, bn);
    bm = __builtin_amdgcn_readfirstlane((int)bm);
    bn = __builtin_amdgcn_readfirstlane((int)bn);
    const int64_t m0 = bm * QM, col0 = bn * QN + wave * QFN * 16;
    // this block's k range: split blockIdx.y of the K dimension
    const int kt0 = (int)(blockIdx.y * p.kt_per_split);
    const int KT = (int)(p.KT - kt0 < p.kt_per_split ? p.KT - kt0 : p.kt_per_split);
    const int64_t K2 = p.K * 2;  // bytes per A row

    // Descriptors: the block's A rows (rows past M read as zero), the wave's
    // weight strips and all group scales.  Loads past the last k-tile (the
    // pipeline's tail) re-read k-tile KT-1 into registers and an LDS slot
    // nothing reads any more, so the loads need no branch.
    const int64_t rows = p.M - m0 < QM ? p.M - m0 : QM;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)p.a + m0 * K2), (short)0, (int)(rows * K2), 0x00020000);
    // strips past N re-read the wave's last strip inside N (or strip 0 when
    // the wave lies wholly past N): their channels are never stored
    const int64_t ntiles = p.N / 16, nt0 = col0 / 16;
    const int64_t bstrips = ntiles - nt0 <= 0 ? 0 : (ntiles - nt0 < QFN ? ntiles - nt0 : QFN);
    const int64_t nb = bstrips ? nt0 : 0, nbs = bstrips ? bstrips : 1;
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w + nb * p.KT * INT4_TILE_BYTES), (short)0, (int)(nbs * p.KT * INT4_TILE_BYTES),
        0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.ep.w_scale, (short)0, (int)(p.KT * p.N * 4), 0x00020000);

    // A DMA: wave w moves rows 4w .. 4w+3 of each of the 8 row strips (u);
    // lane l takes row r = 4w + l/16 and LDS slot l % 16, which holds the
    // row's 16-byte piece (l % 16) ^ r.  The row offset is in the per-lane
    // offset (range-checked: rows past M read zero), the k-tile's in soffset.
    const int ar = 4 * wave + (lane >> 4);
    const uint32_t avoff = (uint32_t)(ar * K2 + (((lane & 15) ^ ar) * 16));
    auto dma_a = [&](int kt) __attribute__((always_inline)) {
        uint8_t* dst = lds + (kt % QS) * QSTAGE + wave * 1024;
        const int ktc = kt0 + (kt < KT ? kt : KT - 1);
#pragma unroll
        for (int u = 0; u < QLD; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(dst + u * 4096), 16,
                                                     (int)(avoff + (uint32_t)(u * 16 * K2)), ktc * 256, 0, 0);
    };
    // Weight tile of strip j, k-tile kt: the lane's 16 packed bytes.
    auto load_b = [&](int kt, u4 (&b)[QFN]) __attribute__((always_inline)) {
        const int ktc = kt0 + (kt < KT ? kt : KT - 1);
#pragma unroll
        for (int j = 0; j < QFN; ++j) {
            const int js = j < nbs ? j : (int)nbs - 1;
            b[j] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rb, lane * 16, (int)((js * p.KT + ktc) * INT4_TILE_BYTES), 0));
        }
    };
    // Group scales of the lane's channels (clamped into N; channels past N
    // are never stored) for k-tile kt.
    int scol[QFN];
#pragma unroll
    for (int j = 0; j < QFN; ++j) {
        const int64_t n = col0 + j * 16 + (lane & 15);
        scol[j] = (int)((n < p.N ? n : p.N - 1) * 4);
    }
    auto load_s = [&](int kt, float (&s)[QFN]) __attribute__((always_inline)) {
        const int ktc = kt0 + (kt < KT ? kt : KT - 1);
#pragma unroll
        for (int j = 0; j < QFN; ++j)
            s[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, scol[j], (int)(ktc * p.N * 4), 0));
    };
    // The lane's operand of row strip i, 8-k chunk c in k-tile kt: row l % 16,
    // k = 32 (l / 16) + 8c .. +7 (the k order of the decoded weight operand).
    const int rr = lane & 15, kg = lane >> 4;
    auto read_a = [&](int kt, int i, int c) __attribute__((always_inline)) {
        return *(const v8h*)(lds + (kt % QS) * QSTAGE + i * 4096 + rr * 256 + (((4 * kg + c) ^ rr) * 16));
    };

    v4f acc[QFM][QFN];
#pragma unroll
    for (int i = 0; i < QFM; ++i)
#pragma unroll
        for (int j = 0; j < QFN; ++j) acc[i][j] = v4f{0, 0, 0, 0};

    // prologue: A stages 0..2, weights and scales of k-tile 0
    u4 bx[QFN], by[QFN];
    float sx[QFN], sy[QFN];
    dma_a(0);
    dma_a(1);
    dma_a(2);
    load_b(0, bx);
    load_s(0, sx);
    wait_vmcnt<0>();
    compiler_fence();
    __syncthreads();
    compiler_fence();
    v8h a[QFM][4];
#pragma unroll
    for (int i = 0; i < QFM; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) a[i][c] = read_a(0, i, c);
    // decoded weight operands (fp16 pairs): the current strip's and the next
    // one's; operand q of a buffer is words 4q .. 4q+3
    uint32_t e0[16], e1[16];
#pragma unroll
    for (int h = 0; h < 8; ++h) dec_part(bx[0], h, e0);
    // the last group sum of a strip pass is folded in the next pass (or the
    // next k-tile's first), once its MFMAs have long completed
    v4f tl = v4f{0, 0, 0, 0};
    float sl = 0.0f;
    int il = 0, jl = 0;  // where tl belongs (compile-time after unrolling)
    (void)il; (void)jl;

    // One k-tile.  On entry: A of kt in a[][], weight strip 0 of kt decoded
    // in e0, raw weights of kt in bc, scales of kt in sc.  Issues the loads
    // of kt+1 (weights bnx, scales sn) and the A stage kt+3.
    auto ktile = [&](int kt, u4 (&bc)[QFN], u4 (&bnx)[QFN], float (&sc)[QFN], float (&sn)[QFN],
                     bool first) __attribute__((always_inline)) {
        // scales of kt and A stage kt+1 have landed (stage kt+2 may be in
        // flight); the barrier publishes every wave's share of stage kt+1
        // and tells that every wave is done with iteration kt-1, whose
        // operand reads were the last ones of the slot stage kt+3 refills
        wait_vmcnt<QLD>();
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        load_b(kt + 1, bnx);
        load_s(kt + 1, sn);
        dma_a(kt + 3);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < QFN; ++j) {
            uint32_t(&cur)[16] = (j & 1) ? e1 : e0;
            uint32_t(&nxt)[16] = (j & 1) ? e0 : e1;
            if (j == QFN - 1) wait_vmcnt<QFN + QLD>();  // weights of kt+1 have landed
            const u4 src = j + 1 < QFN ? bc[j + 1] : bnx[0];
            v4f tp = v4f{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < QFM; ++i) {
                v4f t = v4f{0, 0, 0, 0};
#pragma unroll
                for (int c = 0; c < 4; ++c) t = mfma_f16(a[i][c], as_op(cur, c), t);
                dec_part(src, i, nxt);
                // fold the previous group sum of this wave (the one before
                // in this pass, or the last one of the previous pass)
                if (i > 0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i - 1][j][r] = __builtin_fmaf(tp[r], sc[j], acc[i - 1][j][r]);
                } else if (j > 0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[QFM - 1][j - 1][r] = __builtin_fmaf(tl[r], sl, acc[QFM - 1][j - 1][r]);
                } else if (!first) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[QFM - 1][QFN - 1][r] = __builtin_fmaf(tl[r], sl, acc[QFM - 1][QFN - 1][r]);
                }
                if (j == QFN - 1) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) a[i][c] = read_a(kt + 1, i, c);
                }
                tp = t;
                step_order(j == QFN - 1);
            }
            tl = tp;
            sl = sc[j];
        }
    };
    int kt = 0;
    if (KT > 1) {
        ktile(0, bx, by, sx, sy, true);
        ktile(1, by, bx, sy, sx, false);
        for (kt = 2; kt + 1 < KT; kt += 2) {
            ktile(kt, bx, by, sx, sy, false);
            ktile(kt + 1, by, bx, sy, sx, false);
        }
        if (kt < KT) ktile(kt, bx, by, sx, sy, false);
    } else {
        ktile(0, bx, by, sx, sy, true);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[QFM - 1][QFN - 1][r] = __builtin_fmaf(tl[r], sl, acc[QFM - 1][QFN - 1][r]);

    // ---- epilogue: convert, stage the wave's 128 x 16 QFN tile in LDS, write
    wait_vmcnt<0>();
    compiler_fence();
    __syncthreads();
    uint8_t* band = lds + wave * QEPI_WAVE;
    auto epilogue = [&](auto out_tag) __attribute__((always_inline)) {
        constexpr int OUT = decltype(out_tag)::value;
        constexpr int ESZ = OUT == OUT_F32 ? 4 : 2;
#pragma unroll
        for (int i = 0; i < QFM; ++i)
#pragma unroll
            for (int j = 0; j < QFN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint8_t* d = band + (i * 16 + 4 * kg + r) * QEPI_ROW + (j * 16 + rr) * ESZ;
                    const float v = acc[i][j][r];
                    if constexpr (OUT == OUT_F32) *(float*)d = v;
                    else if constexpr (OUT == OUT_F16) *(uint16_t*)d = (uint16_t)f32_to_f16_bits(v);
                    else *(uint16_t*)d = (uint16_t)f32_to_bf16_bits(v);
                }
        __builtin_amdgcn_wave_barrier();
        if (p.splits > 1)  // fp32 partial sums of this split, summed by the split-K reduce
            copy_out<OUT, QFN>(p, (uint8_t*)p.partial + (int64_t)blockIdx.y * p.M * p.N * 4, p.N, band, m0, col0, lane);
        else
            copy_out<OUT, QFN>(p, (uint8_t*)p.ep.y, p.ep.ldy, band, m0, col0, lane);
    };
    if (p.splits > 1) {
        epilogue(std::integral_constant<int, OUT_F32>{});
        return;
    }
    switch (p.ep.ydt) {
        case OUT_F16: epilogue(std::integral_constant<int, OUT_F16>{}); break;
        case OUT_BF16: epilogue(std::integral_constant<int, OUT_BF16>{}); break;
        default: epilogue(std::integral_constant<int, OUT_F32>{}); break;
    }
}

bool w4a16_tile_fits(int64_t M, int64_t N, int64_t K) {
    (void)M; (void)N;
    // the A row offsets of a block (128 rows of 2K bytes) stay below 2^30
    return K <= (int64_t(1) << 22);
}

template <int QFN>
static hipError_t launch_fn(const LinParams& p, hipStream_t stream) {
    using C = QCfg<QFN>;
    // dynamic LDS above 64 KiB needs the attribute, set once per device
    // (before any graph capture: the first launch is eager)
    static std::atomic<uint64_t> configured{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = uint64_t(1) << (dev & 63);
    if (!(configured.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute((const void*)gemm_w4a16_kernel<QFN>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                C::LDS_ALL);
        if (e != hipSuccess) return e;
        configured.fetch_or(bit, std::memory_order_acq_rel);
    }
    const int64_t blocks = ((p.M + QM - 1) / QM) * ((p.N + C::QN - 1) / C::QN);
    gemm_w4a16_kernel<QFN><<<dim3((unsigned)blocks, (unsigned)p.splits), 64 * QW, C::LDS_ALL, stream>>>(p);
    return hipGetLastError();
}

// Block width and K splits for a shape.  One block per CU at a time, so a
// launch of s splits takes ceil(blocks * s / CUs) rounds of ceil(KT / s)
// k-tiles.  A k-tile of a 128 x 128 block costs 0.6 of a 128 x 256 block's
// (the same A stage, half the weight decode and MFMAs); the fp32 partial
// sums are written and read back once each (8 bytes per output and split),
// and a 128 x 256 block's k-tile takes about as long as the chip moves 9 MB.
// Measured at M = 256 .. 1024 and K = N = 4096 .. 8192 the model picks the
// faster width at every shape or one within 2 % of it (128 x 128 blocks:
// 9-11 % faster at K = N = 4096 and at M = 256, K = N = 5120; up to 32 %
// slower where they need a second round).  At most 8 splits of 4+ k-tiles.
W4A16Plan w4a16_plan(int64_t M, int64_t N, int64_t K) {
    constexpr int64_t CUS = 256;
    constexpr double BYTES_PER_KTILE = 9e6;
    const int64_t kt = K / TILE_K;
    W4A16Plan best{4, 1};
    double best_cost = 0;
    for (int fn : {4, 2}) {
        const int64_t qn = QW * fn * 16, tiles = ((M + QM - 1) / QM) * ((N + qn - 1) / qn);
        const double ktile = fn == 4 ? 1.0 : 0.6;
        for (int s = 1; s <= 8 && (s == 1 || kt / s >= 4); ++s) {
            const double cost = (double)((tiles * s + CUS - 1) / CUS) * ((kt + s - 1) / s) * ktile +
                                (s > 1 ? (double)s * M * N * 8 / BYTES_PER_KTILE : 0.0);
            if (best_cost == 0 || cost < best_cost) {
                best = W4A16Plan{fn, s};
                best_cost = cost;
            }
        }
    }
    return best;
}

int w4a16_tile_splits(int64_t M, int64_t N, int64_t K) { return w4a16_plan(M, N, K).splits; }

hipError_t launch_gemm_w4a16(const LinParams& p, hipStream_t stream) {
    return w4a16_plan(p.M, p.N, p.K).fn == 2 ? launch_fn<2>(p, stream) : launch_fn<4>(p, stream);
}

}  // namespace bql
