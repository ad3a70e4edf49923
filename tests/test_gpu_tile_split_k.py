"""GPU parity of the tile kernels with K split over blocks, against the CPU
oracle.

Shapes with few output tiles (M of a few hundred rows) split K over
blocks: each split's raw sums (fp32, or the exact int32 of W4A8) go to a
partial buffer and a fixed-order reduce applies the epilogue.  Covered:
the exact fp8 kernels with K split (the k-split kernel at M <= 128, the
256-row tile kernel above; dynamic and pre-quantized row-major E4M3 A,
per-channel weights, fp8 output with an output_scale), the fast fp8 kernel
(against its derived bound), W4A8 per channel (int32 accumulators bit for
bit) and per group, and ragged M / N.  The linears are those of vLLM PR
#4118 ("Algorithm"), optimum-quanto PR #241 and QQQ issue #15; float
outputs within |d| <= 5e-3 (|ref| + 1e-2 max|ref|).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import DEV, Weights, assert_close, assert_fast_bound, assert_fp8_out, dev, dev16, host, host_f64, rows_for, say

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu


def _splits(M, N, K, fmt):
    """Split count the library plans, read back from its workspace size."""
    L = bql.lib()
    if fmt == "fp8":
        extra = L.bql_fp8_linear_workspace_size(M, N, K) - 8192 - ((M + 15) // 16) * ((K + 127) // 128) * 2048
    else:
        extra = L.bql_w4a8_linear_workspace_size(M, N, K) - ((M + 15) // 16) * ((K + 127) // 128) * 2048
    return round(extra / (M * N * 4))


@pytest.mark.parametrize("M,N,K", [(128, 4096, 4096), (200, 1040, 8192), (300, 2048, 4096), (17, 784, 14336)])
@pytest.mark.parametrize("prequant", [False, True])
def test_fp8_split_k(M, N, K, prequant):
    assert _splits(M, N, K, "fp8") > 1, "shape must split K"
    say(f"fp8 split K: M={M} N={N} K={K} prequant={prequant} splits={_splits(M, N, K, 'fp8')}")
    W = Weights(131, N + K, N, K, "bf16", True)
    pw = bql.prepack_weight(dev16(W.bits, "bf16"), "fp8_channel")
    a_bits = wl.activation(wl.rng(131, M, N, K), M, K, "bf16", "channels")
    aq_ref, sa_ref = oracle.quant_per_tensor(oracle.decode_input(a_bits, "bf16"))
    a = dev16(a_bits, "bf16")
    if prequant:
        q, sa = bql.quantize_dynamic(a)
        q = q.view(torch.float8_e4m3fn)
        y = bql.fp8_linear(q, pw, a_scale=sa, out_dtype=torch.bfloat16)
        yf = bql.fp8_linear(q, pw, a_scale=sa, out_dtype=torch.bfloat16, fast_accum=True)
    else:
        sa = torch.empty(1, dtype=torch.float32, device=DEV)
        y = bql.fp8_linear(a, pw, a_scale=sa, out_dtype=torch.bfloat16)
        yf = bql.fp8_linear(a, pw, out_dtype=torch.bfloat16, fast_accum=True)
    torch.cuda.synchronize()
    assert host(sa)[0].view(np.uint32) == np.float32(sa_ref).view(np.uint32)
    rows = rows_for(M, 900 + M, 24)
    y_ref = oracle.fp8_linear(aq_ref, sa_ref, W.codes, W.scales, rows=rows)
    assert_close(host_f64(y)[rows], y_ref, f"exact M={M} N={N} K={K}")
    abs_sum = oracle.fp8_acc(aq_ref & 0x7F, W.codes & 0x7F, rows=rows) * np.float64(sa_ref) \
        * W.scales.astype(np.float64)[None, :]
    assert_fast_bound(host_f64(yf)[rows], y_ref, abs_sum, f"fast M={M} N={N} K={K}")
    if not prequant:
        osc = np.float32(np.abs(y_ref).max() / 448.0 * 0.5)  # part of the output saturates
        yq = bql.fp8_linear(a, pw, out_dtype=torch.float8_e4m3fn, output_scale=torch.tensor([osc], device=DEV))
        torch.cuda.synchronize()
        assert_fp8_out(host(yq)[rows], y_ref / np.float64(osc), "  fp8 out x0.5")


@pytest.mark.parametrize("M,N,K", [(256, 4096, 4096), (200, 528, 8192), (130, 1024, 131056 // 16 // 128 * 128 * 16)])
def test_w4a8_split_k_int32_exact(M, N, K):
    assert _splits(M, N, K, "w4a8") > 1, "shape must split K"
    say(f"W4A8 split K: M={M} N={N} K={K} splits={_splits(M, N, K, 'w4a8')}")
    g = wl.rng(132, M, N, K)
    w4 = wl.int4_weight(g, N, K)
    pw = bql.prepack_weight(dev(wl.pack_int4(w4).reshape(N, K // 2)), "int4_channel",
                            scales=dev16(wl.w4a8_channel_scales(g, N), "f16"))
    aq = g.integers(-128, 128, size=(M, K), dtype=np.int8)
    acc = bql.w4a8_linear(dev(aq), None, pw, out_dtype=torch.int32)
    torch.cuda.synchronize()
    rows = rows_for(M, 910 + M, 24)
    assert np.array_equal(host(acc)[rows].astype(np.int64), oracle.w4a8_acc(aq, w4, rows=rows))


@pytest.mark.parametrize("M,N,K", [(256, 4096, 4096), (300, 1040, 8192)])
def test_w4a8_group_split_k(M, N, K):
    assert _splits(M, N, K, "w4a8") > 1, "shape must split K"
    g = wl.rng(133, M, N, K)
    w4 = wl.int4_weight(g, N, K)
    sw = (g.uniform(0.5, 2.0, size=(N, K // 128)) * 2.0 ** -8).astype(np.float32)
    pw = bql.prepack_weight(dev(wl.pack_int4(w4).reshape(N, K // 2)), "int4_group", scales=dev(sw))
    aq = g.integers(-127, 128, size=(M, K), dtype=np.int8)
    sa = g.uniform(1e-3, 1e-1, size=M).astype(np.float32)
    y = bql.w4a8_group_linear(dev(aq), dev(sa), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = rows_for(M, 920 + M, 24)
    assert_close(host_f64(y)[rows], oracle.w4a8_group_linear(aq, sa, w4, sw, rows=rows),
                 f"g128 split K M={M} N={N} K={K}")
