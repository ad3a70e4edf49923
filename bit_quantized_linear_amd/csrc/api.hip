// C ABI of the library: argument checking on the host, then launches.
// Nothing here allocates or synchronizes; see include/bql.h for the
// contract of every entry point.
#include <algorithm>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "bql.h"
#include "kernels.h"
#include "skinny.h"

// Scratch of bql_fp8_linear_noalloc: device memory that the library
// itself holds, one copy per GPU (each device's code object has its own),
// kept until the process ends.  In host code `scratch` is a stand-in, not a
// device address: kernels and copies get the address that
// hipGetSymbolAddress returns on that device.
static __device__ __align__(256) uint8_t scratch[BQL_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

bql_status fail(bql_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

bql_status ok() {
    g_err[0] = '\0';
    return BQL_OK;
}

#define CHECK(expr)                              \
    do {                                         \
        bql_status st__ = (expr);                \
        if (st__ != BQL_OK) return st__;         \
    } while (0)

bql_status need_ptr(const void* p, const char* name) {
    if (!p) return fail(BQL_ERR_NULL, "%s is NULL", name);
    if (((uintptr_t)p) & 15u) return fail(BQL_ERR_ALIGN, "%s is not 16-byte aligned", name);
    return BQL_OK;
}

// Scalars (one fp32) only need natural alignment.
bql_status need_scalar(const void* p, const char* name) {
    if (!p) return fail(BQL_ERR_NULL, "%s is NULL", name);
    if (((uintptr_t)p) & 3u) return fail(BQL_ERR_ALIGN, "%s is not 4-byte aligned", name);
    return BQL_OK;
}

constexpr int64_t MAX_DIM = int64_t(1) << 24;

bql_status need_nk(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0) return fail(BQL_ERR_SHAPE, "N=%lld and K=%lld must be positive", (long long)N, (long long)K);
    if (N % 16 || K % 16)
        return fail(BQL_ERR_SHAPE, "N=%lld and K=%lld must be multiples of 16", (long long)N, (long long)K);
    if (N > MAX_DIM || K > MAX_DIM) return fail(BQL_ERR_SHAPE, "N or K above 2^24");
    return BQL_OK;
}

// The fp8 formats also take 1 <= N < 16 (the small-N path); K stays a
// multiple of 16.
bql_status need_nk_fp8(int64_t N, int64_t K) {
    if (N >= 1 && N < 16) {
        if (K <= 0 || K % 16 || K > MAX_DIM)
            return fail(BQL_ERR_SHAPE, "K=%lld must be a positive multiple of 16", (long long)K);
        return BQL_OK;
    }
    return need_nk(N, K);
}

bql_status need_m(int64_t M) {
    if (M < 0) return fail(BQL_ERR_SHAPE, "M=%lld is negative", (long long)M);
    if (M > (int64_t(1) << 22)) return fail(BQL_ERR_SHAPE, "M above 2^22");
    return BQL_OK;
}

bql_status need_ws(void* ws, size_t have, size_t want) {
    if (want == 0) return BQL_OK;
    if (!ws) return fail(BQL_ERR_WORKSPACE, "workspace of %zu bytes is required", want);
    if (((uintptr_t)ws) & 255u) return fail(BQL_ERR_ALIGN, "workspace is not 256-byte aligned");
    if (have < want) return fail(BQL_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, want);
    return BQL_OK;
}

bool is_f16ish(bql_dtype d) { return d == BQL_F16 || d == BQL_BF16; }

bql_status hip_status(hipError_t e) {
    if (e != hipSuccess) return fail(BQL_ERR_HIP, "HIP: %s", hipGetErrorString(e));
    return ok();
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t ktiles(int64_t K) { return (K + 127) / 128; }

constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch_ptr[MAX_DEVICES];
std::mutex g_scratch_mu;

// The address of the current device's scratch, looked up once per device
// (with that device current) and kept.
bql_status device_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(BQL_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEVICES) return fail(BQL_ERR_ARG, "device %d beyond %d devices", dev, MAX_DEVICES);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return fail(BQL_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                            hipGetErrorString(e));
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return BQL_OK;
}

}  // namespace

extern "C" {

int bql_abi_version(void) { return BQL_ABI_VERSION; }

const char* bql_last_error(void) { return g_err; }

// ------------------------------------------------------------- quantizers

size_t bql_quantize_workspace_size(int64_t numel) {
    (void)numel;
    return bql::QUANT_WS_BYTES;
}

bql_status bql_fp8_quantize_dynamic(const void* x, bql_dtype xdt, int64_t numel, uint8_t* xq,
                                    float* scale_out, void* ws, size_t ws_bytes,
                                    bql_stream stream) {
    if (numel < 0) return fail(BQL_ERR_SHAPE, "numel is negative");
    if (!is_f16ish(xdt)) return fail(BQL_ERR_DTYPE, "x must be BQL_F16 or BQL_BF16");
    CHECK(need_ptr(x, "x"));
    CHECK(need_ptr(xq, "xq"));
    if (scale_out && (((uintptr_t)scale_out) & 3u)) return fail(BQL_ERR_ALIGN, "scale_out misaligned");
    CHECK(need_ws(ws, ws_bytes, bql_quantize_workspace_size(numel)));
    if (numel == 0) return ok();
    return hip_status(bql::launch_quant_dynamic(x, xdt, numel, xq, scale_out, ws, (hipStream_t)stream));
}

bql_status bql_fp8_quantize_static(const void* x, bql_dtype xdt, int64_t numel, const float* scale,
                                   uint8_t* xq, bql_stream stream) {
    if (numel < 0) return fail(BQL_ERR_SHAPE, "numel is negative");
    if (!is_f16ish(xdt)) return fail(BQL_ERR_DTYPE, "x must be BQL_F16 or BQL_BF16");
    CHECK(need_ptr(x, "x"));
    CHECK(need_ptr(xq, "xq"));
    CHECK(need_scalar(scale, "scale"));
    if (numel == 0) return ok();
    return hip_status(bql::launch_quant_static(x, xdt, numel, scale, xq, (hipStream_t)stream));
}

size_t bql_fp8_packed_activation_bytes(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0) return 0;
    return bql::packed_act_bytes(M, K);
}

bql_status bql_fp8_pack_activations(const uint8_t* codes, int64_t M, int64_t K, void* packed,
                                    bql_stream stream) {
    CHECK(need_m(M));
    if (K <= 0 || K % 16 || K > (int64_t(1) << 22))
        return fail(BQL_ERR_SHAPE, "K=%lld must be a positive multiple of 16, at most 2^22", (long long)K);
    if (M == 0) return ok();
    CHECK(need_ptr(codes, "codes"));
    CHECK(need_ptr(packed, "packed"));
    return hip_status(bql::launch_pack_codes(codes, M, K, (uint8_t*)packed, (hipStream_t)stream));
}

bql_status bql_int8_quantize_per_token(const void* x, bql_dtype xdt, int64_t M, int64_t K,
                                       int8_t* xq, float* scales, bql_stream stream) {
    if (!is_f16ish(xdt)) return fail(BQL_ERR_DTYPE, "x must be BQL_F16 or BQL_BF16");
    CHECK(need_m(M));
    if (K <= 0 || K % 16 || K > MAX_DIM) return fail(BQL_ERR_SHAPE, "K must be a positive multiple of 16");
    if (M > 0x7FFFFFFF) return fail(BQL_ERR_SHAPE, "M too large");
    CHECK(need_ptr(x, "x"));
    CHECK(need_ptr(xq, "xq"));
    CHECK(need_ptr(scales, "scales"));
    if (M == 0) return ok();
    return hip_status(bql::launch_int8_per_token(x, xdt, M, K, xq, scales, (hipStream_t)stream));
}

// ------------------------------------------------ RMSNorm + quantization

size_t bql_rmsnorm_quantize_workspace_size(int64_t M) {
    return M > 0 ? bql::rmsnorm_quant_ws_bytes(M) : 0;
}

static bql_status check_rmsnorm_args(const void* x, const void* g, bql_dtype xdt, int64_t M,
                                     int64_t K, float eps, const void* xq, const float* inv_rms) {
    if (!is_f16ish(xdt)) return fail(BQL_ERR_DTYPE, "x must be BQL_F16 or BQL_BF16");
    CHECK(need_m(M));
    if (K <= 0 || K % 16 || K > bql::RMSNORM_MAX_K)
        return fail(BQL_ERR_SHAPE, "K=%lld must be a positive multiple of 16, at most %lld",
                    (long long)K, (long long)bql::RMSNORM_MAX_K);
    if (!(eps > 0.0f) || eps == INFINITY) return fail(BQL_ERR_ARG, "eps must be positive and finite");
    CHECK(need_ptr(x, "x"));
    CHECK(need_ptr(g, "g"));
    CHECK(need_ptr(xq, "xq"));
    if (inv_rms && (((uintptr_t)inv_rms) & 3u)) return fail(BQL_ERR_ALIGN, "inv_rms misaligned");
    return BQL_OK;
}

bql_status bql_rmsnorm_int8_quantize_per_token(const void* x, const void* g, bql_dtype xdt,
                                               int64_t M, int64_t K, float eps, int8_t* xq,
                                               float* scales, float* inv_rms, bql_stream stream) {
    CHECK(check_rmsnorm_args(x, g, xdt, M, K, eps, xq, inv_rms));
    CHECK(need_scalar(scales, "scales"));
    if (M == 0) return ok();
    return hip_status(bql::launch_rmsnorm_int8(x, g, xdt, M, K, eps, xq, scales, inv_rms,
                                               (hipStream_t)stream));
}

bql_status bql_rmsnorm_fp8_quantize_dynamic(const void* x, const void* g, bql_dtype xdt, int64_t M,
                                            int64_t K, float eps, uint8_t* xq, float* scale_out,
                                            float* inv_rms, void* ws, size_t ws_bytes,
                                            bql_stream stream) {
    CHECK(check_rmsnorm_args(x, g, xdt, M, K, eps, xq, inv_rms));
    CHECK(need_scalar(scale_out, "scale_out"));
    CHECK(need_ws(ws, ws_bytes, bql_rmsnorm_quantize_workspace_size(M)));
    if (M == 0) return ok();
    return hip_status(bql::launch_rmsnorm_fp8(x, g, xdt, M, K, eps, xq, scale_out, inv_rms, ws,
                                              (hipStream_t)stream));
}

// ---------------------------------------------------------------- prepack

size_t bql_packed_weight_bytes(int64_t N, int64_t K, bql_wfmt fmt) {
    if (N <= 0 || K <= 0) return 0;
    const size_t tiles = (size_t)((N + 15) / 16) * (size_t)ktiles(K);
    return tiles * ((fmt == BQL_WFMT_INT4_CHANNEL || fmt == BQL_WFMT_INT4_GROUP) ? 1024 : 2048);
}

size_t bql_prepack_workspace_size(int64_t N, int64_t K, bql_wfmt fmt) {
    (void)N; (void)K;
    return fmt == BQL_WFMT_FP8_TENSOR ? bql::QUANT_WS_BYTES : 0;
}

bql_status bql_prepack_weight(const void* w, bql_dtype wdt, int64_t N, int64_t K, bql_wfmt fmt,
                              const void* scales_in, bql_dtype sdt, void* packed,
                              float* scales_out, void* ws, size_t ws_bytes, bql_stream stream) {
    hipStream_t s = (hipStream_t)stream;
    CHECK((fmt == BQL_WFMT_INT4_CHANNEL || fmt == BQL_WFMT_INT4_GROUP) ? need_nk(N, K)
                                                                       : need_nk_fp8(N, K));
    CHECK(need_ptr(w, "w"));
    CHECK(need_ptr(packed, "packed"));
    CHECK(need_ptr(scales_out, "scales_out"));
    if (fmt != BQL_WFMT_FP8_TENSOR && fmt != BQL_WFMT_FP8_CHANNEL && fmt != BQL_WFMT_INT4_CHANNEL &&
        fmt != BQL_WFMT_INT4_GROUP)
        return fail(BQL_ERR_ARG, "unknown weight format %d", (int)fmt);
    if (fmt == BQL_WFMT_INT4_GROUP) {
        if (K % 128) return fail(BQL_ERR_SHAPE, "INT4_GROUP needs K=%lld a multiple of 128", (long long)K);
        if (wdt != BQL_INT4) return fail(BQL_ERR_DTYPE, "INT4_GROUP takes a BQL_INT4 weight");
        if (!scales_in) return fail(BQL_ERR_NULL, "INT4_GROUP needs scales_in");
        if (sdt != BQL_F16 && sdt != BQL_F32) return fail(BQL_ERR_DTYPE, "scales must be BQL_F16 or BQL_F32");
        CHECK(need_scalar(scales_in, "scales_in"));
        if (sdt == BQL_F16 && (((uintptr_t)scales_in) & 1u)) return fail(BQL_ERR_ALIGN, "scales_in misaligned");
        hipError_t e = bql::launch_group_scales(scales_in, sdt == BQL_F16 ? 1 : 3, N, K / 128, scales_out, s);
        if (e == hipSuccess) e = bql::launch_prepack_int4((const uint8_t*)w, N, K, (uint8_t*)packed, s);
        return hip_status(e);
    }
    const int64_t nscales = fmt == BQL_WFMT_FP8_TENSOR ? 1 : N;
    if (scales_in) {
        if (sdt != BQL_F16 && sdt != BQL_F32) return fail(BQL_ERR_DTYPE, "scales must be BQL_F16 or BQL_F32");
        CHECK(need_scalar(scales_in, "scales_in"));
        if (sdt == BQL_F16 && (((uintptr_t)scales_in) & 1u)) return fail(BQL_ERR_ALIGN, "scales_in misaligned");
    }
    if (fmt == BQL_WFMT_INT4_CHANNEL) {
        if (wdt != BQL_INT4) return fail(BQL_ERR_DTYPE, "INT4_CHANNEL takes a BQL_INT4 weight");
        if (!scales_in) return fail(BQL_ERR_NULL, "INT4_CHANNEL needs scales_in");
        hipError_t e = bql::launch_convert_scales(scales_in, sdt == BQL_F16 ? 1 : 3, nscales, scales_out, s);
        if (e == hipSuccess) e = bql::launch_prepack_int4((const uint8_t*)w, N, K, (uint8_t*)packed, s);
        return hip_status(e);
    }
    if (wdt != BQL_F16 && wdt != BQL_BF16 && wdt != BQL_E4M3)
        return fail(BQL_ERR_DTYPE, "FP8 formats take a BQL_F16, BQL_BF16 or BQL_E4M3 weight");
    hipError_t e = hipSuccess;
    if (scales_in) {
        e = bql::launch_convert_scales(scales_in, sdt == BQL_F16 ? 1 : 3, nscales, scales_out, s);
    } else {
        if (wdt == BQL_E4M3) return fail(BQL_ERR_NULL, "an E4M3 weight needs scales_in");
        if (fmt == BQL_WFMT_FP8_TENSOR) {
            CHECK(need_ws(ws, ws_bytes, bql_prepack_workspace_size(N, K, fmt)));
            e = bql::launch_tensor_scale(w, wdt, N * K, 448.0f, scales_out, ws, s);
        } else {
            e = bql::launch_row_scales(w, wdt, N, K, 448.0f, scales_out, s);
        }
    }
    if (e == hipSuccess)
        e = bql::launch_prepack_fp8(w, (int)wdt, N, K, scales_out, fmt == BQL_WFMT_FP8_CHANNEL,
                                    (uint8_t*)packed, s);
    return hip_status(e);
}

bql_status bql_unpack_weight(const void* packed, int64_t N, int64_t K, bql_wfmt fmt, void* out,
                             bql_stream stream) {
    const bool int4 = fmt == BQL_WFMT_INT4_CHANNEL || fmt == BQL_WFMT_INT4_GROUP;
    CHECK(int4 ? need_nk(N, K) : need_nk_fp8(N, K));
    CHECK(need_ptr(packed, "packed"));
    CHECK(need_ptr(out, "out"));
    if (int4)
        return hip_status(bql::launch_unpack_int4((const uint8_t*)packed, N, K, (uint8_t*)out, (hipStream_t)stream));
    if (fmt == BQL_WFMT_FP8_TENSOR || fmt == BQL_WFMT_FP8_CHANNEL)
        return hip_status(bql::launch_unpack_fp8((const uint8_t*)packed, N, K, (uint8_t*)out, (hipStream_t)stream));
    return fail(BQL_ERR_ARG, "unknown weight format %d", (int)fmt);
}

// ---------------------------------------------------------------- linears

// fp8 workspace: [quantizer partials + scale: 8 KiB][Aq, packed operand
// tiles][split-K partials]
size_t bql_fp8_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    const size_t split = std::max(bql::split_ws_bytes(M, N, K, bql::V_FP8), bql::split_ws_bytes(M, N, K, bql::V_FP8X));
    return bql::QUANT_WS_BYTES + align256(bql::packed_act_bytes(M, K)) + align256(split);
}

// N < 16: the small-N kernel reads A where it is (E4M3 codes, or fp16 /
// bf16 cast in registers with the given scale or with amax / 448 from the
// amax partials of one pass over A, kept in the workspace).
static bql_status skinny_fp8_linear(const void* a, bql_dtype adt, const float* a_scale,
                                    float* scale_out, bool static_scale, const void* w_packed,
                                    const float* w_scale, int w_per_channel, int64_t M, int64_t N,
                                    int64_t K, const float* output_scale, void* y, bql_dtype ydt,
                                    bql_accum accum, void* ws, hipStream_t s) {
    int nparts = 0;
    uint32_t* partial = (uint32_t*)ws;
    if (adt != BQL_E4M3 && !static_scale) {
        nparts = bql::launch_amax_partials(a, M * K, partial, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_status(e);
    }
    bql::Epilogue ep;
    ep.y = y;
    ep.ldy = N;
    ep.ydt = ydt;
    ep.a_scale = a_scale;
    ep.w_scale = w_scale;
    ep.w_per_channel = w_per_channel;
    ep.out_scale = output_scale;
    const int src = adt == BQL_E4M3 ? 4 : (adt == BQL_BF16 ? 2 : 1);
    return hip_status(bql::launch_skinny_linear(a, src, (const uint8_t*)w_packed, M, N, K, a_scale,
                                                partial, nparts, scale_out, ep,
                                                accum == BQL_ACCUM_FAST, s));
}

// Argument checks of bql_fp8_linear and bql_fp8_linear_noalloc, all but the
// workspace.
static bql_status check_fp8_linear(const void* a, bql_dtype adt, const float* a_scale,
                                   const void* w_packed, const float* w_scale, int w_per_channel,
                                   int64_t M, int64_t N, int64_t K, const float* output_scale,
                                   const void* y, bql_dtype ydt, bql_accum accum) {
    CHECK(need_m(M));
    CHECK(need_nk_fp8(N, K));
    if (K > (int64_t(1) << 22)) return fail(BQL_ERR_SHAPE, "K above 2^22");
    if (!is_f16ish(adt) && adt != BQL_E4M3 && adt != BQL_E4M3_TILES)
        return fail(BQL_ERR_DTYPE, "A must be BQL_F16, BQL_BF16, BQL_E4M3 or BQL_E4M3_TILES");
    if (adt == BQL_E4M3_TILES && M != 0 && (M <= bql::SMALL_M_MAX || N <= bql::SKINNY_MAX_N))
        return fail(BQL_ERR_SHAPE, "BQL_E4M3_TILES activations need M > %d and N >= 16 (M=%lld N=%lld)",
                    (int)bql::SMALL_M_MAX, (long long)M, (long long)N);
    if (ydt != BQL_F16 && ydt != BQL_BF16 && ydt != BQL_F32 && ydt != BQL_E4M3)
        return fail(BQL_ERR_DTYPE, "Y must be BQL_F16, BQL_BF16, BQL_F32 or BQL_E4M3");
    if (w_per_channel != 0 && w_per_channel != 1) return fail(BQL_ERR_ARG, "w_per_channel must be 0 or 1");
    if (accum != BQL_ACCUM_EXACT && accum != BQL_ACCUM_FAST) return fail(BQL_ERR_ARG, "unknown accum %d", (int)accum);
    if (M == 0) return BQL_OK;
    CHECK(need_ptr(a, "a"));
    CHECK(need_ptr(w_packed, "w_packed"));
    CHECK(need_scalar(w_scale, "w_scale"));
    CHECK(need_ptr(y, "y"));
    if (adt == BQL_E4M3 || adt == BQL_E4M3_TILES) CHECK(need_scalar(a_scale, "a_scale"));
    else if (a_scale && (((uintptr_t)a_scale) & 3u)) return fail(BQL_ERR_ALIGN, "a_scale misaligned");
    if (ydt == BQL_E4M3) CHECK(need_scalar(output_scale, "output_scale"));
    return BQL_OK;
}

// The launches of bql_fp8_linear on checked arguments, M > 0, with a
// workspace of at least bql_fp8_linear_workspace_size(M, N, K) bytes.
static bql_status run_fp8_linear(const void* a, bql_dtype adt, float* a_scale, const void* w_packed,
                                 const float* w_scale, int w_per_channel, int64_t M, int64_t N,
                                 int64_t K, const float* output_scale, void* y, bql_dtype ydt,
                                 bql_accum accum, void* ws, hipStream_t s) {
    if (N <= bql::SKINNY_MAX_N)
        return skinny_fp8_linear(a, adt, a_scale, a_scale, false, w_packed, w_scale, w_per_channel,
                                 M, N, K, output_scale, y, ydt, accum, ws, s);
    char* wsb = (char*)ws;
    uint8_t* aq = (uint8_t*)(wsb + bql::QUANT_WS_BYTES);
    char* part = wsb + bql::QUANT_WS_BYTES + align256(bql::packed_act_bytes(M, K));
    const int variant = accum == BQL_ACCUM_FAST ? bql::V_FP8 : bql::V_FP8X;
    const bool codes = adt == BQL_E4M3 || adt == BQL_E4M3_TILES;
    if (!codes && bql::fused_small_m(M, N, K)) {
        // one launch: the small-M kernel quantizes A itself
        bql::LinearArgs la;
        la.variant = variant;
        la.a = a;
        la.w = (const uint8_t*)w_packed;
        la.M = M;
        la.N = N;
        la.K = K;
        la.y = y;
        la.ydt = ydt;
        la.a_scale = nullptr;
        la.w_scale = w_scale;
        la.w_per_channel = w_per_channel;
        la.out_scale = output_scale;
        la.fused = 1;
        la.xdt = adt;
        la.scale_out = a_scale;
        la.scale_ws = (float*)(wsb + 4096);
        return hip_status(bql::launch_linear(la, part, bql::split_ws_bytes(M, N, K, variant), s));
    }
    const float* sa = a_scale;
    // pre-quantized A is read row-major where it is by the kernels that read
    // it that way at full speed (small M, the k-split exact tile kernel)
    // and packed A (BQL_E4M3_TILES) where it is by every tile kernel
    const bool direct = adt == BQL_E4M3 && bql::reads_rowmajor_a(variant, M, N, K);
    hipError_t e = hipSuccess;
    if (!codes) {
        e = bql::launch_quant_dynamic_packed(a, adt, M, K, aq, a_scale, wsb, s);
        sa = (const float*)(wsb + 4096);
    } else if (adt == BQL_E4M3 && !direct) {
        e = bql::launch_pack_codes((const uint8_t*)a, M, K, aq, s);
    }
    if (e != hipSuccess) return hip_status(e);
    bql::LinearArgs la;
    la.variant = variant;
    la.a = direct || adt == BQL_E4M3_TILES ? a : aq;
    la.a_rowmajor = direct ? 1 : 0;
    la.w = (const uint8_t*)w_packed;
    la.M = M;
    la.N = N;
    la.K = K;
    la.y = y;
    la.ydt = ydt;
    la.a_scale = sa;
    la.w_scale = w_scale;
    la.w_per_channel = w_per_channel;
    la.out_scale = output_scale;
    return hip_status(bql::launch_linear(la, part, bql::split_ws_bytes(M, N, K, variant), s));
}

bql_status bql_fp8_linear(const void* a, bql_dtype adt, float* a_scale, const void* w_packed,
                          const float* w_scale, int w_per_channel, int64_t M, int64_t N, int64_t K,
                          const float* output_scale, void* y, bql_dtype ydt, bql_accum accum,
                          void* ws, size_t ws_bytes, bql_stream stream) {
    CHECK(check_fp8_linear(a, adt, a_scale, w_packed, w_scale, w_per_channel, M, N, K, output_scale,
                           y, ydt, accum));
    if (M == 0) return ok();
    CHECK(need_ws(ws, ws_bytes, bql_fp8_linear_workspace_size(M, N, K)));
    return run_fp8_linear(a, adt, a_scale, w_packed, w_scale, w_per_channel, M, N, K, output_scale,
                          y, ydt, accum, ws, (hipStream_t)stream);
}

bql_status bql_fp8_linear_noalloc(const void* a, bql_dtype adt, float* a_scale,
                                  const void* w_packed, const float* w_scale, int w_per_channel,
                                  int64_t M, int64_t N, int64_t K, const float* output_scale,
                                  void* y, bql_dtype ydt, bql_accum accum, bql_stream stream) {
    CHECK(check_fp8_linear(a, adt, a_scale, w_packed, w_scale, w_per_channel, M, N, K, output_scale,
                           y, ydt, accum));
    if (M == 0) return ok();
    const size_t need = bql_fp8_linear_workspace_size(M, N, K);
    if (need > BQL_NOALLOC_SCRATCH_BYTES)
        return fail(BQL_ERR_SHAPE,
                    "M=%lld N=%lld K=%lld needs %zu bytes of scratch, above the %zu bytes of "
                    "bql_fp8_linear_noalloc (use bql_fp8_linear with a workspace)",
                    (long long)M, (long long)N, (long long)K, need, (size_t)BQL_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    CHECK(device_scratch(&ws));
    return run_fp8_linear(a, adt, a_scale, w_packed, w_scale, w_per_channel, M, N, K, output_scale,
                          y, ydt, accum, ws, (hipStream_t)stream);
}

bql_status bql_fp8_linear_static(const void* a, bql_dtype adt, const float* a_scale,
                                 const void* w_packed, const float* w_scale, int w_per_channel,
                                 int64_t M, int64_t N, int64_t K, const float* output_scale,
                                 void* y, bql_dtype ydt, bql_accum accum, void* ws,
                                 size_t ws_bytes, bql_stream stream) {
    hipStream_t s = (hipStream_t)stream;
    CHECK(need_m(M));
    CHECK(need_nk_fp8(N, K));
    if (K > (int64_t(1) << 22)) return fail(BQL_ERR_SHAPE, "K above 2^22");
    if (!is_f16ish(adt)) return fail(BQL_ERR_DTYPE, "A must be BQL_F16 or BQL_BF16");
    if (ydt != BQL_F16 && ydt != BQL_BF16 && ydt != BQL_F32 && ydt != BQL_E4M3)
        return fail(BQL_ERR_DTYPE, "Y must be BQL_F16, BQL_BF16, BQL_F32 or BQL_E4M3");
    if (w_per_channel != 0 && w_per_channel != 1) return fail(BQL_ERR_ARG, "w_per_channel must be 0 or 1");
    if (accum != BQL_ACCUM_EXACT && accum != BQL_ACCUM_FAST) return fail(BQL_ERR_ARG, "unknown accum %d", (int)accum);
    if (M == 0) return ok();
    CHECK(need_ptr(a, "a"));
    CHECK(need_scalar(a_scale, "a_scale"));
    CHECK(need_ptr(w_packed, "w_packed"));
    CHECK(need_scalar(w_scale, "w_scale"));
    CHECK(need_ptr(y, "y"));
    if (ydt == BQL_E4M3) CHECK(need_scalar(output_scale, "output_scale"));
    CHECK(need_ws(ws, ws_bytes, bql_fp8_linear_workspace_size(M, N, K)));
    if (N <= bql::SKINNY_MAX_N)
        return skinny_fp8_linear(a, adt, a_scale, nullptr, true, w_packed, w_scale, w_per_channel,
                                 M, N, K, output_scale, y, ydt, accum, ws, s);

    char* wsb = (char*)ws;
    uint8_t* aq = (uint8_t*)(wsb + bql::QUANT_WS_BYTES);
    char* part = wsb + bql::QUANT_WS_BYTES + align256(bql::packed_act_bytes(M, K));
    const int variant = accum == BQL_ACCUM_FAST ? bql::V_FP8 : bql::V_FP8X;
    bql::LinearArgs la;
    la.variant = variant;
    la.w = (const uint8_t*)w_packed;
    la.M = M;
    la.N = N;
    la.K = K;
    la.y = y;
    la.ydt = ydt;
    la.a_scale = a_scale;
    la.w_scale = w_scale;
    la.w_per_channel = w_per_channel;
    la.out_scale = output_scale;
    if (bql::fused_small_m(M, N, K)) {
        // one launch: the small-M kernel casts A with the given scale itself
        la.a = a;
        la.fused = 1;
        la.xdt = adt;
        la.given_scale = a_scale;
        return hip_status(bql::launch_linear(la, part, bql::split_ws_bytes(M, N, K, variant), s));
    }
    hipError_t e = bql::launch_quant_static_packed(a, adt, M, K, a_scale, aq, s);
    if (e != hipSuccess) return hip_status(e);
    la.a = aq;
    return hip_status(bql::launch_linear(la, part, bql::split_ws_bytes(M, N, K, variant), s));
}

size_t bql_w8a16_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return align256(bql::split_ws_bytes(M, N, K, bql::V_W8A16));
}

bql_status bql_w8a16_linear(const void* a, const void* w_packed, const float* w_scales, int64_t M,
                            int64_t N, int64_t K, void* y, bql_dtype ydt, void* ws, size_t ws_bytes,
                            bql_stream stream) {
    CHECK(need_m(M));
    CHECK(need_nk(N, K));
    if (M > (int64_t(65535) * 16)) return fail(BQL_ERR_SHAPE, "M above 1048560");
    if (ydt != BQL_F16 && ydt != BQL_BF16 && ydt != BQL_F32)
        return fail(BQL_ERR_DTYPE, "Y must be BQL_F16, BQL_BF16 or BQL_F32");
    if (M == 0) return ok();
    CHECK(need_ptr(a, "a"));
    CHECK(need_ptr(w_packed, "w_packed"));
    CHECK(need_ptr(w_scales, "w_scales"));
    CHECK(need_ptr(y, "y"));
    CHECK(need_ws(ws, ws_bytes, bql_w8a16_linear_workspace_size(M, N, K)));
    bql::LinearArgs la;
    la.variant = bql::V_W8A16;
    la.a = a;
    la.w = (const uint8_t*)w_packed;
    la.M = M;
    la.N = N;
    la.K = K;
    la.y = y;
    la.ydt = ydt;
    la.a_scale = nullptr;
    la.w_scale = w_scales;
    la.w_per_channel = 1;
    la.out_scale = nullptr;
    return hip_status(bql::launch_linear(la, ws, ws_bytes, (hipStream_t)stream));
}

// W4A8 workspace: [Aq, packed operand tiles][split-K partials]
size_t bql_w4a8_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return align256(bql::packed_act_bytes(M, K)) + align256(bql::split_ws_bytes(M, N, K, bql::V_W4A8));
}

bql_status bql_w4a8_linear(const int8_t* aq, const float* a_scales, const void* w_packed,
                           const float* w_scales, int64_t M, int64_t N, int64_t K, void* y,
                           bql_dtype ydt, void* ws, size_t ws_bytes, bql_stream stream) {
    CHECK(need_m(M));
    CHECK(need_nk(N, K));
    // 16 * |acc| <= 16 * 128 * 8 * K must stay inside int32: K <= 131056
    // gives at most 2^31 - 2^18 (all products -128 * -8)
    if (K > 131056) return fail(BQL_ERR_SHAPE, "K above 131056 could overflow the int32 accumulator");
    if (ydt != BQL_F16 && ydt != BQL_BF16 && ydt != BQL_F32 && ydt != BQL_I32)
        return fail(BQL_ERR_DTYPE, "Y must be BQL_F16, BQL_BF16, BQL_F32 or BQL_I32");
    if (M == 0) return ok();
    CHECK(need_ptr(aq, "aq"));
    CHECK(need_ptr(w_packed, "w_packed"));
    CHECK(need_ptr(y, "y"));
    if (ydt != BQL_I32) {
        CHECK(need_ptr(a_scales, "a_scales"));
        CHECK(need_ptr(w_scales, "w_scales"));
    }
    CHECK(need_ws(ws, ws_bytes, bql_w4a8_linear_workspace_size(M, N, K)));
    uint8_t* aq_ws = (uint8_t*)ws;
    // the small-M path reads the row-major int8 A where it is
    const bool direct = bql::use_small_m(bql::V_W4A8, M, N, K);
    if (!direct) {
        hipError_t e = bql::launch_pack_codes((const uint8_t*)aq, M, K, aq_ws, (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e);
    }
    bql::LinearArgs la;
    la.variant = bql::V_W4A8;
    la.a = direct ? (const void*)aq : (const void*)aq_ws;
    la.a_rowmajor = direct ? 1 : 0;
    la.w = (const uint8_t*)w_packed;
    la.M = M;
    la.N = N;
    la.K = K;
    la.y = y;
    la.ydt = ydt;
    la.a_scale = a_scales;
    la.w_scale = w_scales;
    la.w_per_channel = 1;
    la.out_scale = nullptr;
    char* part = (char*)ws + align256(bql::packed_act_bytes(M, K));
    return hip_status(bql::launch_linear(la, part, bql::split_ws_bytes(M, N, K, bql::V_W4A8),
                                         (hipStream_t)stream));
}

bql_status bql_w4a8_group_linear(const int8_t* aq, const float* a_scales, const void* w_packed,
                                 const float* w_scales, int64_t M, int64_t N, int64_t K,
                                 int64_t group_size, void* y, bql_dtype ydt, void* ws,
                                 size_t ws_bytes, bql_stream stream) {
    CHECK(need_m(M));
    CHECK(need_nk(N, K));
    if (group_size != 128) return fail(BQL_ERR_ARG, "group_size must be 128");
    if (K % 128 || K / 128 > bql::W4A8G_MAX_KT)
        return fail(BQL_ERR_SHAPE, "K=%lld must be a multiple of 128, at most %d", (long long)K,
                    128 * bql::W4A8G_MAX_KT);
    if (N * (K / 128) * 4 >= (int64_t(1) << 31))
        return fail(BQL_ERR_SHAPE, "N * K/128 group scales must fit in 2 GiB");
    if (ydt != BQL_F16 && ydt != BQL_BF16 && ydt != BQL_F32)
        return fail(BQL_ERR_DTYPE, "Y must be BQL_F16, BQL_BF16 or BQL_F32");
    if (M == 0) return ok();
    CHECK(need_ptr(aq, "aq"));
    CHECK(need_ptr(w_packed, "w_packed"));
    CHECK(need_ptr(y, "y"));
    CHECK(need_ptr(a_scales, "a_scales"));
    CHECK(need_ptr(w_scales, "w_scales"));
    CHECK(need_ws(ws, ws_bytes, bql_w4a8_linear_workspace_size(M, N, K)));
    uint8_t* aq_ws = (uint8_t*)ws;
    // the small-M path reads the row-major int8 A where it is
    const bool direct = bql::use_small_m(bql::V_W4A8G, M, N, K);
    if (!direct) {
        hipError_t e = bql::launch_pack_codes((const uint8_t*)aq, M, K, aq_ws, (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e);
    }
    bql::LinearArgs la;
    la.variant = bql::V_W4A8G;
    la.a = direct ? (const void*)aq : (const void*)aq_ws;
    la.a_rowmajor = direct ? 1 : 0;
    la.w = (const uint8_t*)w_packed;
    la.M = M;
    la.N = N;
    la.K = K;
    la.y = y;
    la.ydt = ydt;
    la.a_scale = a_scales;
    la.w_scale = w_scales;
    la.w_per_channel = 1;
    la.out_scale = nullptr;
    char* part = (char*)ws + align256(bql::packed_act_bytes(M, K));
    return hip_status(bql::launch_linear(la, part, bql::split_ws_bytes(M, N, K, bql::V_W4A8G),
                                         (hipStream_t)stream));
}

size_t bql_w4a16_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return align256(bql::w4a16_ws_bytes(M, N, K));
}

bql_status bql_w4a16_group_linear(const void* a, const void* w_packed, const float* w_scales,
                                  int64_t M, int64_t N, int64_t K, int64_t group_size, void* y,
                                  bql_dtype ydt, void* ws, size_t ws_bytes, bql_stream stream) {
    CHECK(need_m(M));
    CHECK(need_nk(N, K));
    if (M > (int64_t(65535) * 16)) return fail(BQL_ERR_SHAPE, "M above 1048560");
    if (group_size != 128) return fail(BQL_ERR_ARG, "group_size must be 128");
    if (K % 128) return fail(BQL_ERR_SHAPE, "K=%lld must be a multiple of 128", (long long)K);
    if (N * (K / 128) * 4 >= (int64_t(1) << 31))
        return fail(BQL_ERR_SHAPE, "N * K/128 group scales must fit in 2 GiB");
    if (ydt != BQL_F16 && ydt != BQL_BF16 && ydt != BQL_F32)
        return fail(BQL_ERR_DTYPE, "Y must be BQL_F16, BQL_BF16 or BQL_F32");
    if (M == 0) return ok();
    CHECK(need_ptr(a, "a"));
    CHECK(need_ptr(w_packed, "w_packed"));
    CHECK(need_ptr(w_scales, "w_scales"));
    CHECK(need_ptr(y, "y"));
    CHECK(need_ws(ws, ws_bytes, bql_w4a16_linear_workspace_size(M, N, K)));
    bql::LinearArgs la;
    la.variant = bql::V_W4A16G;
    la.a = a;
    la.w = (const uint8_t*)w_packed;
    la.M = M;
    la.N = N;
    la.K = K;
    la.y = y;
    la.ydt = ydt;
    la.a_scale = nullptr;
    la.w_scale = w_scales;
    la.w_per_channel = 1;
    la.out_scale = nullptr;
    return hip_status(bql::launch_linear(la, ws, ws_bytes, (hipStream_t)stream));
}

}  // extern "C"
