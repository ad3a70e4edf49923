// Host-side launchers of the gfx950 kernels (internal to the library).
// Every launcher only enqueues work on `stream` and returns the HIP status
// of the launch; argument checking happens before, in the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bql {

// ---------------------------------------------------------------- quant.hip
// Partial amax blocks used by the per-tensor reductions.
int amax_blocks(int64_t numel);
// Bytes of workspace the per-tensor quantizer needs (partials + scale).
constexpr size_t QUANT_WS_BYTES = 8192;
// Dynamic per-tensor E4M3 quantization.  ws holds the partials (first
// 4096 bytes) and the scale (at byte 4096); scale_out may be null.
hipError_t launch_quant_dynamic(const void* x, int xdt, int64_t numel, uint8_t* xq,
                                float* scale_out, void* ws, hipStream_t stream);
// Bytes of the packed 8-bit activation layout (16 x 128 operand tiles).
size_t packed_act_bytes(int64_t M, int64_t K);
// M at and below which the linears run the small-M (streaming) kernels,
// which read A row-major; above it the tile kernels take packed A.
constexpr int64_t SMALL_M_MAX = 16;
// Dynamic per-tensor E4M3 of a row-major [M, K] activation, written in the
// packed layout the linear kernels read.
hipError_t launch_quant_dynamic_packed(const void* x, int xdt, int64_t M, int64_t K, uint8_t* xq,
                                       float* scale_out, void* ws, hipStream_t stream);
// Row-major 8-bit codes [M, K] (E4M3 or int8) -> packed layout.
hipError_t launch_pack_codes(const uint8_t* src, int64_t M, int64_t K, uint8_t* dst,
                             hipStream_t stream);
hipError_t launch_quant_static(const void* x, int xdt, int64_t numel, const float* scale,
                               uint8_t* xq, hipStream_t stream);
// E4M3 with a given scale of a row-major [M, K] activation, written in the
// packed layout the linear kernels read.
hipError_t launch_quant_static_packed(const void* x, int xdt, int64_t M, int64_t K,
                                      const float* scale, uint8_t* xq, hipStream_t stream);
hipError_t launch_int8_per_token(const void* x, int xdt, int64_t M, int64_t K, int8_t* xq,
                                 float* scales, hipStream_t stream);
// amax over numel 16-bit values -> scale = amax / qmax (1 if amax == 0)
// written to *scale; uses ws partials.
hipError_t launch_tensor_scale(const void* x, int xdt, int64_t numel, float qmax,
                               float* scale, void* ws, hipStream_t stream);

// ----------------------------------------------------------- norm_quant.hip
// RMSNorm fused with per-token int8 (one launch) or per-tensor E4M3 (two
// launches; ws holds one maximum per row-kernel block, at most M, and the M
// inverse RMS values).  K <= 32768.
constexpr int64_t RMSNORM_MAX_K = 32768;
size_t rmsnorm_quant_ws_bytes(int64_t M);
hipError_t launch_rmsnorm_int8(const void* x, const void* g, int xdt, int64_t M, int64_t K,
                               float eps, int8_t* xq, float* scales, float* inv_rms,
                               hipStream_t stream);
hipError_t launch_rmsnorm_fp8(const void* x, const void* g, int xdt, int64_t M, int64_t K,
                              float eps, uint8_t* xq, float* scale_out, float* inv_rms, void* ws,
                              hipStream_t stream);

// -------------------------------------------------------------- prepack.hip
hipError_t launch_row_scales(const void* w, int wdt, int64_t N, int64_t K, float qmax,
                             float* scales, hipStream_t stream);
hipError_t launch_convert_scales(const void* s, int sdt, int64_t count, float* out,
                                 hipStream_t stream);
// wdt: 1 f16, 2 bf16, 4 e4m3 codes.  per_row selects scales[n] over scales[0].
hipError_t launch_prepack_fp8(const void* w, int wdt, int64_t N, int64_t K, const float* scales,
                              int per_row, uint8_t* packed, hipStream_t stream);
hipError_t launch_prepack_int4(const uint8_t* w, int64_t N, int64_t K, uint8_t* packed,
                               hipStream_t stream);
hipError_t launch_unpack_fp8(const uint8_t* packed, int64_t N, int64_t K, uint8_t* out,
                             hipStream_t stream);
hipError_t launch_unpack_int4(const uint8_t* packed, int64_t N, int64_t K, uint8_t* out,
                              hipStream_t stream);

// ----------------------------------------------------------------- linears
// V_FP8: E4M3 x E4M3 on the fp8 matrix cores (the hardware's fp8 dot
//        accumulation); V_FP8X: E4M3 x E4M3 decoded losslessly to fp16 and
//        summed exactly on the f16 matrix cores; V_W8A16: fp16 x E4M3 on the
//        f16 matrix cores; V_W4A8: int8 x int4 on the int8 matrix cores.
//        V_W4A16G: fp16 x int4 (weight-only) with one scale per output
//        channel and 128-k group, each group summed on the f16 matrix cores;
//        V_W4A8G: V_W4A8 with one scale per output channel and 128-k group,
//        applied to each k-tile's exact int32 sum, summed in fp32.
enum Variant { V_FP8 = 0, V_W8A16 = 1, V_W4A8 = 2, V_FP8X = 3, V_W4A8G = 4, V_W4A16G = 5 };
// Longest K of the per-group path, in 128-k tiles (its block stages the
// group scales of all k-tiles in LDS).
constexpr int W4A8G_MAX_KT = 128;

struct LinearArgs {
    int variant;
    const void* a;          // fp8 codes / fp16 / int8, [M, K] row-major
    const uint8_t* w;       // packed tiles
    int64_t M, N, K;
    // epilogue
    void* y;
    int ydt;
    const float* a_scale;   // fp8: device scalar; w4a8: [M]
    const float* w_scale;   // V_W4A8G, V_W4A16G: group scales [K/128][N]
    int w_per_channel;
    const float* out_scale;
    // fused small-M fp8: A is row-major fp16/bf16 and is quantized in-kernel
    int fused = 0;
    int xdt = 0;
    float* scale_out = nullptr;  // optional copy of sA for the caller
    float* scale_ws = nullptr;   // sA in the workspace (read by the split-K reduce)
    // 8-bit A is read row-major [M, K] where it is (no repack launch); only
    // where reads_rowmajor_a() holds
    int a_rowmajor = 0;
    // fused small-M fp8 with a static activation scale (no amax): sA = *given_scale
    const float* given_scale = nullptr;
};

// Whether an fp8 call with dynamic quantization runs the fused small-M kernel.
bool fused_small_m(int64_t M, int64_t N, int64_t K);

// Workspace bytes the small-M (split-K) path may use at this shape.
size_t small_m_ws_bytes(int64_t M, int64_t N, int64_t K, int variant);
// Workspace bytes of the per-group W4A16 linear at this shape (split-K
// partial sums of the streaming or the tile kernel).
size_t w4a16_ws_bytes(int64_t M, int64_t N, int64_t K);
// Workspace bytes of a linear's split-K partial sums at this shape, for the
// kernel that runs it (streaming or tile): 0 when K is not split.
size_t split_ws_bytes(int64_t M, int64_t N, int64_t K, int variant);
// Which path runs: true for the streaming small-M kernels.
bool use_small_m(int variant, int64_t M, int64_t N, int64_t K);
// Whether the kernel that runs at this shape reads 8-bit A row-major at full
// speed: the small-M kernels and the k-split exact tile kernel.  The other
// tile kernels are faster on packed operand tiles even with the repack.
bool reads_rowmajor_a(int variant, int64_t M, int64_t N, int64_t K);
hipError_t launch_linear(const LinearArgs& args, void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace bql
