// Launchers of the small-N fp8 linear (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"

namespace bql {

// Widest N the small-N path serves (one 16-channel strip, N < 16).
constexpr int64_t SKINNY_MAX_N = 15;

// Per-group W4A8 scales [N][G] (sdt 1 = fp16, 3 = fp32) -> [G][N] fp32
// (prepack.hip).
hipError_t launch_group_scales(const void* s, int sdt, int64_t N, int64_t G, float* out,
                               hipStream_t stream);

// Per-block amax partials of numel 16-bit values (quant.hip); returns the
// number of partials written (at most 1024).
int launch_amax_partials(const void* x, int64_t numel, uint32_t* partial, hipStream_t stream);

// Y[m, n] = (sA * sW[n]) * sum_k dec(Aq[m, k]) dec(Wq[n, k]) for n < N <= 15.
// a: row-major [M, K]: E4M3 codes (adt = 4) or fp16 / bf16 (adt = IN_F16 /
// IN_BF16), cast in registers as E4M3(x / sA).  sA: *scale when nparts == 0
// (the given scale of codes or of a static cast); otherwise amax / 448 from
// the nparts amax partials (written to scale_out when that is not null).
// w: the packed weight (one strip, channels >= N zero).  fast: the fp8
// matrix cores' own accumulation.
hipError_t launch_skinny_linear(const void* a, int adt, const uint8_t* w, int64_t M, int64_t N,
                                int64_t K, const float* scale, const uint32_t* partial, int nparts,
                                float* scale_out, const Epilogue& ep, bool fast, hipStream_t stream);

}  // namespace bql
