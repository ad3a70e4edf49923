// Exact fp8 tile kernel for large M: Y = (sA*sW[n]) * sum_k dec(Aq)*dec(Wq)
// (vLLM PR #4118, the torch._scaled_mm micro-benchmark) with every product
// formed exactly and summed in fp32.
//
// The E4M3 codes are widened losslessly to fp16 in registers (every finite
// E4M3 value is an fp16 value) and multiplied on the f16 matrix cores
// (v_mfma_f32_16x16x32_f16), whose products are exact.  The fp8 matrix-core
// instruction would be twice as fast but adds each run of 8 products in a
// narrow fixed-point window, which misses the stated tolerance on outlier
// inputs.  So the matrix-core ceiling of this kernel is the f16 one, and the
// fp8 -> f16 conversion is vector-ALU work on top of it.
//
// Organisation (gfx950: 4 SIMDs per CU, 160 KiB LDS per CU):
//   * A block computes 256 rows x 32 fn columns (fn = 2 .. 8, chosen per
//     shape with the K split by exact_plan below).  Blocks up to 192 columns
//     run eight waves of 64 rows, two per SIMD; wider ones four waves of 128
//     rows, one per SIMD, each holding a 128 x 16 fn sub-tile in the
//     accumulation registers (256 fp32 per lane at fn = 8), so that each
//     fp8 -> f16 conversion of A feeds fn MFMAs.
//   * Both operands are in HBM in the 16-row x 128-k operand-tile layout
//     (weights by prepack, activations by the quantizer).  A stage of the LDS
//     ring is one half of a k-tile (64 k) of the block's 16 A strips and its
//     B strips, up to 32 KiB, moved by LDS-DMA (buffer_load ... lds, 1 KiB
//     per wave instruction, no VGPR staging); four stages are in flight.
//   * Per wave, a half-step is two MFMA k-slices of 8 k per lane.  Slice 0
//     multiplies with the B operands decoded during the previous half-step,
//     and meanwhile decodes B's slice 1 and reads the next half-step's raw B
//     from LDS; slice 1 multiplies, decodes the next half-step's B slice 0
//     and reads the next raw A.  Each A operand is decoded one row strip
//     ahead of its MFMAs.  So LDS reads are consumed a whole slice (64 MFMAs)
//     after they are issued, and the conversions run between MFMAs.
//   * One barrier per half-step: it publishes the next stage's DMA and frees
//     the ring slot the next DMA overwrites.
//   * Output tiles are handed to the 8 XCDs in contiguous ranges (each XCD's
//     L2 then holds the B strips its blocks share), and the epilogue stages
//     each 16-row band in LDS and writes it with 16-byte stores.
#include <atomic>
#include <type_traits>

#include "linear_common.h"

namespace bql {

namespace {

constexpr int XB = 256;                    // block rows
constexpr int XSTRIPS = XB / 16;           // 16-row A strips per block
constexpr int XS = 4;                      // LDS ring depth (stages)
constexpr int XCOLS = 128;                 // most columns a wave owns (8 strips)
constexpr int XEPI_ROW = XCOLS * 4 + 16;   // epilogue row: up to 128 fp32 values, padded

// Geometry of a block of 256 rows x 2 FN 16-column B strips: WM waves along
// M (each XF = 16 / WM A strips) times 2 along N (each FN B strips).  A
// stage holds the block's 16 A strips and its B strips rounded up to whole
// DMA rounds (one slot per wave per round); slots past the block's B
// strips are loaded out of range (zeros, no memory access) and never read.
template <int FN, int WM>
struct XCfg {
    static constexpr int XW = 2 * WM;                     // waves per block
    static constexpr int XF = XSTRIPS / WM;               // A strips per wave
    static constexpr int BPS = (FN + XF - 1) / XF;        // B strips a step of a slice handles
    static constexpr int BSLOTS = (2 * FN + XW - 1) / XW * XW;
    static constexpr int SLOTS = XSTRIPS + BSLOTS;
    static constexpr int STAGE = SLOTS * 1024;            // half a k-tile of every slot
    static constexpr int LD = SLOTS / XW;                 // DMA instructions per wave per stage
    static constexpr int LDS = XS * STAGE;
    static constexpr int EPI_ROWS = XF / 2 * 16;          // rows a wave stages per epilogue pass
    static constexpr int EPI_WAVE = EPI_ROWS * XEPI_ROW;
    static constexpr int EPI_SCALES = XW * EPI_WAVE;      // then XCOLS column scales per wave
    static constexpr int LDS_EPI = EPI_SCALES + XW * XCOLS * 4;
    static constexpr int LDS_ALL = LDS > LDS_EPI ? LDS : LDS_EPI;
    static_assert(FN <= 8 && (WM == 2 || WM == 4), "shape");
    static_assert(LD * 2 < 64 && LD <= XF, "vmcnt range; one DMA instruction per step");
    static_assert(LDS <= EPI_SCALES, "the column scales lie past the ring");
};

// Eight E4M3 codes -> eight fp16 of the same values (4 conversions).
__device__ __forceinline__ v8h dec8(uint32_t d0, uint32_t d1) { return e4m3x8_to_f16(d0, d1); }

// Compiler-only fence: keeps LDS reads and writes on their side of the
// workgroup barriers (the LDS-DMA writes are not visible to the compiler).
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Scales ROWS staged rows of accumulators (16 FN fp32 values each, XEPI_ROW
// bytes apart) by their column's sA * sW[n] (colsc), converts them to the
// output dtype OUT and writes them with 16-byte stores: a lane handles
// 16 / (output size) consecutive columns per store, all of a pass's stores
// unrolled so that their LDS reads overlap.  N is a multiple of 16, so a
// store's columns lie all inside or all outside N.  Roundings as the other
// kernels' epilogue: nearest even to fp16 / bf16, E4M3 of fp32(Y / output_scale).
// RAW: the unscaled fp32 sums, into a split-K partial buffer.
template <int OUT, int FN, int ROWS, bool RAW = false>
__device__ __forceinline__ void store_rows_t(const LinParams& p, void* dst, int64_t ld, const float* band,
                                             const float* colsc, int64_t rbase, int64_t col0,
                                             int lane) {
    static_assert(!RAW || OUT == OUT_F32, "partials are fp32");
    constexpr int ESZ = OUT == OUT_E4M3 ? 1 : (OUT == OUT_F32 ? 4 : 2);
    constexpr int PER = 16 / ESZ, CHUNKS = FN * 16 / PER, ITEMS = ROWS * CHUNKS, ITERS = (ITEMS + 63) / 64;
    // E4M3 output: y / output_scale as the IEEE quotient (quot_f32, from the
    // fp64 reciprocal), two codes per conversion instruction
    const double inv = OUT == OUT_E4M3 ? 1.0 / (double)*p.ep.out_scale : 1.0;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int q = lane + 64 * it;
        if (ITEMS % 64 != 0 && q >= ITEMS) break;
        const int row = q / CHUNKS, c0 = (q % CHUNKS) * PER;
        const int64_t m = rbase + row, n = col0 + c0;
        const float* src = band + row * (XEPI_ROW / 4) + c0;
        float y[PER];
#pragma unroll
        for (int e = 0; e < PER; e += 4) {
            const v4f x = *(const v4f*)(src + e), c = *(const v4f*)(colsc + c0 + e);
#pragma unroll
            for (int t = 0; t < 4; ++t) y[e + t] = RAW ? x[t] : c[t] * x[t];
        }
        uint32_t w[4] = {0, 0, 0, 0};
        if constexpr (OUT == OUT_BF16) {
#pragma unroll
            for (int e = 0; e < PER; e += 2) w[e / 2] = f32x2_to_bf16x2(y[e], y[e + 1]);
        } else if constexpr (OUT == OUT_E4M3) {
#pragma unroll
            for (int e = 0; e < PER; e += 2)
                w[e / 4] |= e4m3_encode2(quot_f32(y[e], inv), quot_f32(y[e + 1], inv)) << (8 * (e % 4));
        } else {
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                uint32_t b;
                if constexpr (OUT == OUT_F32) b = __float_as_uint(y[e]);
                else b = f32_to_f16_bits(y[e]);
                w[e * ESZ / 4] |= b << (8 * ((e * ESZ) % 4));
            }
        }
        if (m < p.M && n < p.N) *(u4*)((uint8_t*)dst + (m * ld + n) * ESZ) = u4{w[0], w[1], w[2], w[3]};
    }
}

// Instruction order of one A strip's step of a slice, for the scheduler:
// each of its FN MFMAs is followed by one VALU instruction (the conversions
// of the next operands; measured on gfx950, 16x16x32 MFMAs issue fastest
// with one VALU instruction between consecutive ones, faster than back to
// back), then the step's other conversions, its LDS reads and, in slice 0,
// its DMA instruction.  Nothing moves across steps: a conversion pulled
// forward from a later step could wait on an LDS read issued just before it.
// VALUS: the step's conversions (4 per 8-code operand).
template <bool DMA, int FN, int VALUS, int DS>
__device__ __forceinline__ void interleave() {
    constexpr int MFMA = 0x008, VALU = 0x002, DS_READ = 0x100, VMEM_READ = 0x020;
#pragma unroll
    for (int k = 0; k < FN; ++k) {
        __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(VALU, 1, 0);
    }
    if constexpr (FN < VALUS) __builtin_amdgcn_sched_group_barrier(VALU, VALUS - FN, 0);
    __builtin_amdgcn_sched_group_barrier(DS_READ, DS, 0);
    if constexpr (DMA) __builtin_amdgcn_sched_group_barrier(VMEM_READ, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace

// FN: 16-column B strips per wave (8: 256 x 256 blocks, 7: 256 x 224, ...,
// 2: 256 x 64).  WM = 2: four waves of 128 rows, one per SIMD; WM = 4: eight
// waves of 64 rows, two per SIMD (each with at most 256 registers).  With
// p.splits > 1, block column blockIdx.y takes k-tiles [blockIdx.y *
// kt_per_split, + kt_per_split) and writes its raw fp32 sums to that
// split's partial buffer; the split-K reduce applies the epilogue.
template <int FN, int WM>
__global__ __launch_bounds__(128 * WM) __attribute__((amdgpu_waves_per_eu(WM / 2, WM / 2)))
void gemm_exact_kernel(LinParams p) {
    using C = XCfg<FN, WM>;
    constexpr int XW = C::XW, XF = C::XF, BPS = C::BPS;
    constexpr int BN = 32 * FN;  // block columns
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // the wave index and the tile coordinates (whose 64-bit divisions run on
    // the vector ALU) are uniform: read them as such, so that the DMA
    // addresses built from them stay scalar
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int64_t bm, bn;
    tile_coords(blockIdx.x, (p.M + XB - 1) / XB, (p.N + BN - 1) / BN, bm, bn);
    bm = __builtin_amdgcn_readfirstlane((int)bm);
    bn = __builtin_amdgcn_readfirstlane((int)bn);
    const int64_t mt0 = bm * XSTRIPS, nt0 = bn * (2 * FN);
    const int64_t mtiles = (p.M + 15) / 16, ntiles = p.N / 16;
    const int KT = (int)p.KT;  // the operands' k-tile stride
    // this block's k-tiles: [kt0, kt0 + KTL)
    const int kt0 = (int)blockIdx.y * (int)p.kt_per_split;
    const int KTL = KT - kt0 < (int)p.kt_per_split ? KT - kt0 : (int)p.kt_per_split;

    // Buffer descriptors over this block's strips: rows past M and channels
    // past N lie beyond them and read as zero.
    const int64_t a_strips = mtiles - mt0 < XSTRIPS ? mtiles - mt0 : XSTRIPS;
    const int64_t b_strips = ntiles - nt0 < 2 * FN ? ntiles - nt0 : 2 * FN;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)p.a + mt0 * p.KT * 2048), (short)0, (int)(a_strips * p.KT * 2048),
        0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w + nt0 * p.KT * 2048), (short)0, (int)(b_strips * p.KT * 2048), 0x00020000);

    // Half-step s = k-tile kt0 + s/2, half s%2, goes to ring slot s % XS.
    // Slot q of a stage holds A strip q (q < 16) or B strip q - 16; wave w
    // moves slots w + XW i, i < LD: its A strips, then its B strips.  The first
    // stages are issued whole (issue), the later ones one instruction per
    // step of the main loop (issue_one), also past the last stage: those get
    // an out-of-range offset (zeros, no memory access) into a slot nothing
    // reads any more, so that every half-step issues the same loads.
    auto issue = [&](int s) __attribute__((always_inline)) {
        const int kt = kt0 + (s >> 1), h = s & 1;
        uint8_t* base = lds + (s % XS) * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::LD; ++i) {
            const int slot = wave + XW * i;
            if (i < XSTRIPS / XW) {  // A slots
                const int off = (slot * KT + kt) * 2048 + h * 1024 + lane * 16;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(base + slot * 1024), 16, off,
                                                         0, 0, 0);
            } else {
                const int off = ((slot - XSTRIPS) * KT + kt) * 2048 + h * 1024 + lane * 16;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(base + slot * 1024), 16, off,
                                                         0, 0, 0);
            }
        }
    };
    const int H = 2 * KTL;
    const int lane16 = lane * 16;
    auto issue_one = [&](int s, int i) __attribute__((always_inline)) {
        if (i >= C::LD) return;
        const int kt = kt0 + (s >> 1), h = s & 1, slot = wave + XW * i;
        uint8_t* dst = lds + (s % XS) * C::STAGE + slot * 1024;
        // uniform part of the offset; past the last stage it lies beyond
        // every descriptor's range (at most 2^30 bytes), so all lanes read 0
        constexpr int A_LD = XSTRIPS / XW;  // the first A_LD instructions move A slots
        const bool is_a = i < A_LD;
        const int strip = is_a ? slot : slot - XSTRIPS;
        const int uoff = s < H ? (strip * KT + kt) * 2048 + h * 1024 : 0x7FFF0000;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? ra : rb, (lds_ptr_t)dst, 16, lane16 + uoff, 0, 0, 0);
    };
    // A lane's 16 bytes of strip i of this wave (A) / j (B) in half-step s:
    // bytes 0-7 feed MFMA slice 0, bytes 8-15 slice 1 (same k map for both).
    auto read_a = [&](int s, int i) __attribute__((always_inline)) {
        return *(const u4*)(lds + (s % XS) * C::STAGE + (wm * XF + i) * 1024 + lane * 16);
    };
    auto read_b = [&](int s, int j) __attribute__((always_inline)) {
        return *(const u4*)(lds + (s % XS) * C::STAGE + (XSTRIPS + wn * FN + j) * 1024 + lane * 16);
    };

    const int64_t m0 = bm * XB + wm * XF * 16, col0 = bn * BN + wn * FN * 16;
    // sA * sW[n] of the wave's 128 output columns (one value per tensor),
    // kept in LDS past the operand ring until the epilogue
    float* colsc = (float*)(lds + C::EPI_SCALES) + wave * XCOLS;
    if (lane < 16) {
        const float sa = *p.ep.a_scale;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t n = col0 + j * 16 + lane;
            colsc[j * 16 + lane] = sa * p.ep.w_scale[p.ep.w_per_channel ? (n < p.N ? n : p.N - 1) : 0];
        }
    }
    v4f acc[XF][FN];
#pragma unroll
    for (int i = 0; i < XF; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0, 0, 0, 0};

#pragma unroll
    for (int s = 0; s < XS - 1; ++s)
        if (s < H) issue(s);
    // stage 0 is in (stages issued after it: min(H - 1, 2)); H >= 2
    if (H >= 3) wait_vmcnt<2 * C::LD>();
    else if (H == 2) wait_vmcnt<C::LD>();
    else wait_vmcnt<0>();
    compiler_fence();
    lds_barrier();
    compiler_fence();

    u4 ra_[XF], rb_[FN];   // raw codes of the current (A) / current-then-next (B) half-step
    v8h b0[FN], b1[FN];    // decoded B slices 0 and 1
#pragma unroll
    for (int i = 0; i < XF; ++i) ra_[i] = read_a(0, i);
#pragma unroll
    for (int j = 0; j < FN; ++j) rb_[j] = read_b(0, j);
#pragma unroll
    for (int j = 0; j < FN; ++j) b0[j] = dec8(rb_[j][0], rb_[j][1]);

    // One half-step.  The next half-step's raw operands are read from LDS
    // during it (after the last half-step these reads see a slot nothing
    // writes any more, and their values are never used).  Decodes are
    // written before the MFMAs that run beside them, so that their results
    // do not take the registers of operands those MFMAs still read.
    auto half_step = [&](int s) __attribute__((always_inline)) {
        // this wave's DMA of stage s+1 has landed (stage s+2 may be
        // pending); the barrier makes every wave's share visible and tells
        // that every wave has consumed the slot that stage s+3 overwrites
        // (its reads completed in half-step s-1, when their data was
        // decoded), so it needs no wait on LDS reads
        if (s + 2 < H) wait_vmcnt<C::LD>();
        else wait_vmcnt<0>();
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();

        // slice 0: MFMAs on b0; decode B slice 1 and read the next raw B
        // (BPS strips per step); one DMA instruction of stage s+3 per step
        v8h a = dec8(ra_[0][0], ra_[0][1]);
#pragma unroll
        for (int i = 0; i < XF; ++i) {
            v8h an;
            if (i + 1 < XF) an = dec8(ra_[i + 1][0], ra_[i + 1][1]);
            else an = dec8(ra_[0][2], ra_[0][3]);  // slice 1's first A operand
#pragma unroll
            for (int j = i * BPS; j < (i + 1) * BPS && j < FN; ++j) b1[j] = dec8(rb_[j][2], rb_[j][3]);
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma_f16(a, b0[j], acc[i][j]);
#pragma unroll
            for (int j = i * BPS; j < (i + 1) * BPS && j < FN; ++j) rb_[j] = read_b(s + 1, j);
            issue_one(s + 3, i);
            a = an;
            interleave<true, FN, 4 + 4 * BPS, BPS>();
        }
        // slice 1: MFMAs on b1; read the next raw A; decode the next B slice 0
#pragma unroll
        for (int i = 0; i < XF; ++i) {
            v8h an = a;
            if (i + 1 < XF) an = dec8(ra_[i + 1][2], ra_[i + 1][3]);
            ra_[i] = read_a(s + 1, i);
#pragma unroll
            for (int j = i * BPS; j < (i + 1) * BPS && j < FN; ++j) b0[j] = dec8(rb_[j][0], rb_[j][1]);
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma_f16(a, b1[j], acc[i][j]);
            a = an;
            interleave<false, FN, 4 + 4 * BPS, 1>();
        }
    };
    // the last half-step is written out after the loop: with it inside, the
    // compiler does not keep the accumulators in place across the back edge
    for (int s = 0; s + 1 < H; ++s) half_step(s);
    half_step(H - 1);

    // ---- epilogue, in two passes of half the wave's rows: the fp32
    // accumulators are staged in LDS straight from the accumulation
    // registers (compile-time indices), then scaled by their column's
    // sA * sW[n], converted and written with 16-byte stores
    wait_vmcnt<0>();
    compiler_fence();
    __syncthreads();
    float* band = (float*)(lds + wave * C::EPI_WAVE);
    auto stage = [&](auto ib_tag) __attribute__((always_inline)) {
        constexpr int IB = decltype(ib_tag)::value;
#pragma unroll
        for (int i = 0; i < XF / 2; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    band[(i * 16 + 4 * (lane >> 4) + r) * (XEPI_ROW / 4) + j * 16 + (lane & 15)] =
                        acc[IB + i][j][r];
    };
    // the staged rows and scales are written and read back by this wave only
    auto epilogue = [&](auto out_tag, auto raw_tag, void* dst, int64_t ld) __attribute__((always_inline)) {
        constexpr int OUT = decltype(out_tag)::value;
        constexpr bool RAW = decltype(raw_tag)::value;
        stage(std::integral_constant<int, 0>{});
        __builtin_amdgcn_wave_barrier();
        store_rows_t<OUT, FN, C::EPI_ROWS, RAW>(p, dst, ld, band, colsc, m0, col0, lane);
        __builtin_amdgcn_wave_barrier();
        stage(std::integral_constant<int, XF / 2>{});
        __builtin_amdgcn_wave_barrier();
        store_rows_t<OUT, FN, C::EPI_ROWS, RAW>(p, dst, ld, band, colsc, m0 + C::EPI_ROWS, col0, lane);
    };
    if (p.splits > 1) {
        float* part = (float*)p.partial + (int64_t)blockIdx.y * p.M * p.N;
        epilogue(std::integral_constant<int, OUT_F32>{}, std::true_type{}, part, p.N);
        return;
    }
    const std::false_type scaled;
    void* y = p.ep.y;
    const int64_t ldy = p.ep.ldy;
    switch (p.ep.ydt) {
        case OUT_BF16: epilogue(std::integral_constant<int, OUT_BF16>{}, scaled, y, ldy); break;
        case OUT_F16: epilogue(std::integral_constant<int, OUT_F16>{}, scaled, y, ldy); break;
        case OUT_F32: epilogue(std::integral_constant<int, OUT_F32>{}, scaled, y, ldy); break;
        default: epilogue(std::integral_constant<int, OUT_E4M3>{}, scaled, y, ldy); break;
    }
}

template <int FN, int WM>
static hipError_t launch_fn(const LinParams& p, hipStream_t stream) {
    using C = XCfg<FN, WM>;
    // dynamic LDS above 64 KiB needs the attribute, set once per device
    // (before any graph capture: the first launch is eager)
    static std::atomic<uint64_t> configured{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = uint64_t(1) << (dev & 63);
    if (!(configured.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute((const void*)gemm_exact_kernel<FN, WM>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_ALL);
        if (e != hipSuccess) return e;
        configured.fetch_or(bit, std::memory_order_acq_rel);
    }
    const int64_t blocks = ((p.M + XB - 1) / XB) * ((p.N + 32 * FN - 1) / (32 * FN));
    gemm_exact_kernel<FN, WM><<<dim3((unsigned)blocks, (unsigned)p.splits), 64 * C::XW, C::LDS_ALL, stream>>>(p);
    return hipGetLastError();
}

// Block width (fn strips of 16 columns per wave) and K splits for a shape,
// from a cost model in microseconds fitted to timings of every (fn, splits)
// at M = 200 .. 4096 on Llama-shaped N x K (MI355X).  One block per CU at a
// time, so a launch takes full rounds of CUS blocks and a tail round (whose
// k-tiles run a little faster: fewer busy CUs, higher clock); a k-tile of a
// block costs a fixed part (the A side: its 16 strips' DMA, reads and
// conversions) and a part per B strip; K splits add the fp32 partials'
// write and read and the reduce launch.  At M = 128 (one 128-row tile) the
// 128-row kernels measured 6-19 % faster; from M = 200 up this kernel was as
// fast or faster (up to 32 % at M = 512, N = 28672).
ExactPlan exact_plan(int64_t M, int64_t N, int64_t K) {
    constexpr int64_t CUS = 256;
    constexpr double KTILE_US = 0.76, KTILE_US_PER_FN = 0.25, BLOCK_US = 1.3, TAIL_SPEED = 0.95;
    constexpr double PARTIAL_BYTES_PER_US = 6.0e6, REDUCE_US = 6.0;
    constexpr int FNS[] = {8, 7, 6, 4, 3, 2};
    ExactPlan best{0, 1};
    if (M <= 128) return best;
    const int64_t KT = (K + 127) / 128, mt = (M + XB - 1) / XB;
    double best_us = 0;
    for (int fn : FNS) {
        const int64_t tiles = mt * ((N + 32 * fn - 1) / (32 * fn));
        const double ktile = KTILE_US + KTILE_US_PER_FN * fn;
        for (int s = 1; s <= 4; ++s) {
            const int64_t per = (KT + s - 1) / s, splits = (KT + per - 1) / per;
            if (splits != s || (s > 1 && per < 4)) continue;
            const int64_t full = tiles * s / CUS, tail = tiles * s % CUS;
            double us = full * (BLOCK_US + per * ktile);
            if (tail) us += BLOCK_US + per * ktile * (TAIL_SPEED + (1 - TAIL_SPEED) * tail / CUS);
            if (s > 1) us += (double)s * M * N * 8 / PARTIAL_BYTES_PER_US + REDUCE_US;
            if (best.fn == 0 || us < best_us) {
                best = ExactPlan{fn, s};
                best_us = us;
            }
        }
    }
    return best;
}

// Blocks of 256 x 64 .. 256 x 192 run eight waves (two per SIMD), wider
// ones four: measured on MI355X at M = 1024 and 4096, eight waves are 1-12 %
// faster for fn <= 6 and up to 2.5 % slower for fn = 7 and 8.
hipError_t launch_gemm_exact(const LinParams& p, const ExactPlan& plan, hipStream_t stream) {
    switch (plan.fn) {
        case 8: return launch_fn<8, 2>(p, stream);
        case 7: return launch_fn<7, 2>(p, stream);
        case 6: return launch_fn<6, 4>(p, stream);
        case 4: return launch_fn<4, 4>(p, stream);
        case 3: return launch_fn<3, 4>(p, stream);
        case 2: return launch_fn<2, 4>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bql
