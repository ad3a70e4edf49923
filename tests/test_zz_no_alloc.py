"""GPU check of bql_fp8_linear_noalloc, the allocation-free variant of
bql_fp8_linear for callers that cannot allocate (graph capture, serving
loops, harnesses that forbid hipMalloc).

Both entry points run the same kernels on the same inputs, the first with
the caller's workspace and the second with the library's own per-GPU
scratch, so outputs and activation scales must be identical bit for bit.
Two calls in a row, the second with a smaller input, check that nothing of
the first call's scratch content leaks into the second.  The outputs are
also held to the oracle's tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import DEV, Weights, assert_close, dev16, host, host_f64, rows_for, say

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu

# (M, N, K): the tile path with dynamic quantization, then smaller calls
# through the small-M streaming path and the fused one-launch path
SEQUENCES = [
    [(1024, 4096, 4096), (200, 1024, 1024)],
    [(16, 6144, 4096), (4, 1024, 1024)],
    [(640, 2048, 14336), (1, 4096, 14336)],
]


def _case(M, N, K, idx, per_channel=False):
    W = Weights(93, idx, N, K, "bf16", per_channel)
    pw = bql.prepack_weight(dev16(W.bits, "bf16"), "fp8_channel" if per_channel else "fp8_tensor")
    a_bits = wl.activation(wl.rng(93, idx, M, 3), M, K, "bf16", "channels")
    a = dev16(a_bits, "bf16")
    aq_ref, sa_ref = oracle.quant_per_tensor(oracle.decode_input(a_bits, "bf16"))
    return W, pw, a, aq_ref, sa_ref


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_matches_workspace_call(seq):
    for step, (M, N, K) in enumerate(SEQUENCES[seq]):
        say(f"noalloc seq {seq} step {step}: M={M} N={N} K={K}")
        W, pw, a, aq_ref, sa_ref = _case(M, N, K, 10 * seq + step)
        sa_ws = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
        sa_na = torch.full((1,), -2.0, dtype=torch.float32, device=DEV)
        y_ws = bql.fp8_linear(a, pw, a_scale=sa_ws, out_dtype=torch.bfloat16)
        y_na = bql.fp8_linear_noalloc(a, pw, a_scale=sa_na, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(host(y_na), host(y_ws)), "outputs differ from bql_fp8_linear"
        assert host(sa_na).view(np.uint32)[0] == host(sa_ws).view(np.uint32)[0]
        assert host(sa_na)[0] == np.float32(sa_ref)
        rows = rows_for(M, 300 + M, 24)
        y_ref = oracle.fp8_linear(aq_ref, sa_ref, W.codes, W.scales, rows=rows)
        assert_close(host_f64(y_na)[rows], y_ref, f"noalloc M={M} N={N} K={K}")


def test_noalloc_prequantized_per_channel_fp8_out():
    # pre-quantized E4M3 A, per-channel weight scales, fp8 output with an
    # output_scale; then a smaller call with bf16 output
    for step, (M, N, K, fp8_out) in enumerate([(512, 3072, 8192, True), (48, 1024, 2048, False)]):
        say(f"noalloc prequantized step {step}: M={M} N={N} K={K}")
        W, pw, a, aq_ref, sa_ref = _case(M, N, K, 40 + step, per_channel=True)
        q, sa = bql.quantize_dynamic(a)
        qv = q.view(torch.float8_e4m3fn)
        if fp8_out:
            osc = torch.tensor([0.05], dtype=torch.float32, device=DEV)
            y_ws = bql.fp8_linear(qv, pw, a_scale=sa, out_dtype=torch.float8_e4m3fn, output_scale=osc)
            y_na = bql.fp8_linear_noalloc(qv, pw, a_scale=sa, out_dtype=torch.float8_e4m3fn,
                                          output_scale=osc)
        else:
            y_ws = bql.fp8_linear(qv, pw, a_scale=sa, out_dtype=torch.bfloat16)
            y_na = bql.fp8_linear_noalloc(qv, pw, a_scale=sa, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(host(y_na), host(y_ws)), "outputs differ from bql_fp8_linear"
        assert np.array_equal(host(q), aq_ref)
        if not fp8_out:
            rows = rows_for(M, 400 + M, 24)
            y_ref = oracle.fp8_linear(aq_ref, sa_ref, W.codes, W.scales, rows=rows)
            assert_close(host_f64(y_na)[rows], y_ref, f"noalloc prequantized M={M}")


def test_noalloc_packed_activations():
    # pre-packed E4M3 A (BQL_E4M3_TILES) through the exact tile kernel with
    # K split, then a smaller call at a narrower block width
    for step, (M, N, K) in enumerate([(520, 4208, 8000), (300, 2048, 4096)]):
        say(f"noalloc packed step {step}: M={M} N={N} K={K}")
        W, pw, a, aq_ref, sa_ref = _case(M, N, K, 50 + step)
        q, sa = bql.quantize_dynamic(a)
        pa = bql.pack_activations(q)
        y_ws = bql.fp8_linear(pa, pw, a_scale=sa, out_dtype=torch.bfloat16)
        y_na = bql.fp8_linear_noalloc(pa, pw, a_scale=sa, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(host(y_na), host(y_ws)), "outputs differ from bql_fp8_linear"
        rows = rows_for(M, 450 + M, 16)
        y_ref = oracle.fp8_linear(aq_ref, sa_ref, W.codes, W.scales, rows=rows)
        assert_close(host_f64(y_na)[rows], y_ref, f"noalloc packed M={M}")


def test_noalloc_refuses_oversized_call():
    M, N, K = 8192, 4096, 8192
    assert bql.fp8_linear_workspace_size(M, N, K) > bql.NOALLOC_SCRATCH_BYTES
    # full-size buffers, so that even a launch would stay in bounds; the
    # call must fail on the host before launching anything
    a = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    pw = bql.PackedWeight(torch.zeros(bql.packed_weight_bytes(N, K, "fp8_tensor"), dtype=torch.uint8,
                                      device=DEV),
                          torch.ones(1, dtype=torch.float32, device=DEV), N, K, "fp8_tensor")
    with pytest.raises(bql.BQLError, match="BQL_ERR_SHAPE"):
        bql.fp8_linear_noalloc(a, pw)
