"""GPU parity of the fp8 linear at N < 16 (the MoE router of the vLLM FP8
quantization-schema RFC discussion: gate_proj with 8 experts, which FP8
GEMMs that need N divisible by 16 leave in 16-bit) against the CPU oracle.

Weights are packed in one 16-channel strip with the channels past N zero;
outputs, scales and every caller-visible buffer have exactly N columns.
Float outputs within the stated tolerance; activation scales identical;
unpacked codes identical; the fp8 matrix cores' own accumulation within its
derived bound.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import (DEV, assert_close, assert_fast_bound, assert_fp8_out, dev, dev16, host,
                     host_f64, rows_for, say)

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu


def _weight(N, K, dtype, seed):
    g = wl.rng(96, seed, N, K)
    bits = wl.weight(g, N, K, dtype)
    return bits, oracle.decode_input(bits, dtype)


# (M, N, K): router shapes (8 experts on Llama-3-8B / Mixtral-like hidden
# sizes), every M regime, ragged M, odd N, minimal K; ragged M with a
# partial last k-tile (A is loaded in whole rows of a tile and regrouped, so
# rows past M and chunks past K must read as zero in that mapping too)
CASES = [(1, 8, 4096), (16, 8, 4096), (128, 8, 4096), (1024, 8, 4096), (4096, 8, 4096),
         (1000, 8, 5120), (37, 1, 4096), (300, 3, 1024), (64, 15, 8192), (5, 8, 16),
         (33, 12, 48), (2048, 2, 14336), (19, 8, 400), (260, 5, 4112)]


@pytest.mark.parametrize("M,N,K", CASES)
@pytest.mark.parametrize("per_channel", [False, True])
def test_small_n_dynamic(M, N, K, per_channel):
    wb, wf = _weight(N, K, "bf16", 1)
    pw = bql.prepack_weight(dev16(wb, "bf16"), "fp8_channel" if per_channel else "fp8_tensor")
    codes, scales = oracle.quant_per_row(wf) if per_channel else oracle.quant_per_tensor(wf)
    scales = np.atleast_1d(np.asarray(scales, dtype=np.float32))
    assert np.array_equal(host(bql.unpack_weight(pw)), codes), "unpacked codes differ"
    assert np.array_equal(host(pw.scales).view(np.uint32), scales.view(np.uint32))
    ab = wl.activation(wl.rng(96, 2, M, K), M, K, "bf16", "channels")
    sa = torch.empty(1, dtype=torch.float32, device=DEV)
    y = bql.fp8_linear(dev16(ab, "bf16"), pw, a_scale=sa, out_dtype=torch.bfloat16)
    yf = bql.fp8_linear(dev16(ab, "bf16"), pw, out_dtype=torch.float32, fast_accum=True)
    torch.cuda.synchronize()
    assert y.shape == (M, N)
    aq, s_ref = oracle.quant_per_tensor(oracle.decode_input(ab, "bf16"))
    assert host(sa)[0].view(np.uint32) == np.float32(s_ref).view(np.uint32)
    rows = rows_for(M, 300 + M, 256)
    ref = oracle.fp8_linear(aq, s_ref, codes, scales, rows=rows)
    assert_close(host_f64(y)[rows], ref, f"M={M} N={N} K={K} per_channel={per_channel}")
    sw = scales if scales.size == N else np.full(N, scales[0], dtype=np.float32)
    abs_sum = oracle.fp8_acc(aq & 0x7F, codes & 0x7F, rows=rows) * np.float64(s_ref) \
        * sw.astype(np.float64)[None, :]
    assert_fast_bound(host_f64(yf)[rows], ref, abs_sum, f"M={M} N={N} fast accumulation")


@pytest.mark.parametrize("M,K", [(1, 4096), (256, 4096), (37, 400)])
def test_small_n_prequantized_static_and_fp8_out(M, K):
    N = 8
    wb, wf = _weight(N, K, "f16", 3)
    pw = bql.prepack_weight(dev16(wb, "f16"), "fp8_tensor")
    codes, sw = oracle.quant_per_tensor(wf)
    ab = wl.activation(wl.rng(96, 4, M, K), M, K, "f16", "entries")
    x = oracle.decode_input(ab, "f16")
    aq, s_ref = oracle.quant_per_tensor(x)
    ref = oracle.fp8_linear(aq, s_ref, codes, np.array([sw], np.float32))
    # pre-quantized E4M3 input
    y = bql.fp8_linear(dev(aq).view(torch.float8_e4m3fn), pw,
                       a_scale=torch.tensor([s_ref], device=DEV), out_dtype=torch.float16)
    # static scale (2x the amax scale: nothing saturates)
    s2 = np.float32(s_ref * np.float32(2))
    ys = bql.fp8_linear_static(dev16(ab, "f16"), pw, torch.tensor([s2], device=DEV),
                               out_dtype=torch.float32)
    # fp8 output with an output scale
    osc = np.float32(np.abs(ref).max() / 448.0)
    yq = bql.fp8_linear(dev16(ab, "f16"), pw, out_dtype=torch.float8_e4m3fn,
                        output_scale=torch.tensor([osc], device=DEV))
    torch.cuda.synchronize()
    assert_close(host_f64(y), ref, f"M={M} pre-quantized")
    aq2 = oracle.quant_with_scales(x, np.array([s2], np.float32))
    assert_close(host_f64(ys), oracle.fp8_linear(aq2, s2, codes, np.array([sw], np.float32)),
                 f"M={M} static scale")
    assert_fp8_out(host(yq), ref / np.float64(osc), f"M={M} fp8 out")


def test_small_n_e4m3_weight_input_and_determinism():
    # codes given with per-channel scales (prepack of an E4M3 weight)
    N, K, M = 8, 1024, 64
    g = np.random.Generator(np.random.PCG64(5))
    codes = g.integers(0, 256, size=(N, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00  # no NaN codes
    sc = (g.uniform(0.5, 2.0, N) * 2.0 ** -8).astype(np.float32)
    pw = bql.prepack_weight(dev(codes).view(torch.float8_e4m3fn), "fp8_channel", scales=dev(sc))
    assert np.array_equal(host(bql.unpack_weight(pw)), codes)
    ab = wl.activation(wl.rng(96, 6, M, K), M, K, "bf16", "none")
    a = dev16(ab, "bf16")
    y1 = bql.fp8_linear(a, pw, out_dtype=torch.float32)
    y2 = bql.fp8_linear(a, pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    aq, s_ref = oracle.quant_per_tensor(oracle.decode_input(ab, "bf16"))
    assert_close(host_f64(y1), oracle.fp8_linear(aq, s_ref, codes, sc), "E4M3 weight, N=8")
    say("  N=8 from E4M3 codes: deterministic")
