"""GPU parity of the weight prepack (bit-exact codes and scales).

Per-tensor weight scale after load (vLLM PR #4118, "Algorithm"), per-channel
scales (optimum-quanto PR #241), caller-given fp16 scales (the W8A16
decode workload), E4M3 checkpoint codes passed through, and int4 packing
(QQQ issue #15).  The packed layout is private; bql_unpack_weight returns
the logical codes, which must equal the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import DEV, dev, dev16, host, say

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["fp8_tensor", "fp8_channel"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N,K", [(48, 144), (1024, 1024), (4096, 4096), (160, 272)])
def test_prepack_fp8_computed_scales(fmt, dtype, N, K):
    g = wl.rng(7, N, K)
    bits = wl.weight(g, N, K, dtype)
    pw = bql.prepack_weight(dev16(bits, dtype), fmt)
    codes = host(bql.unpack_weight(pw))
    wf = oracle.decode_input(bits, dtype)
    if fmt == "fp8_tensor":
        q, s = oracle.quant_per_tensor(wf)
        s = np.array([s], dtype=np.float32)
    else:
        q, s = oracle.quant_per_row(wf)
    assert np.array_equal(host(pw.scales).view(np.uint32), s.view(np.uint32))
    assert np.array_equal(codes, q)
    assert pw.packed.numel() == bql.packed_weight_bytes(N, K, fmt)


@pytest.mark.parametrize("fmt", ["fp8_tensor", "fp8_channel"])
def test_prepack_fp8_nan_weight(fmt):
    # a NaN weight makes the amax of its tensor (per tensor) or of its row
    # (per channel) NaN: that scale is NaN and its codes are NaN codes, of
    # either sign (a division's NaN has no fixed sign); the other rows keep
    # their exact codes and scales
    N, K = 160, 272
    g = wl.rng(7, N, K, 1)
    w = oracle.decode_input(wl.weight(g, N, K, "bf16"), "bf16").astype(np.float32)
    w[37, 100] = np.nan
    bits = wl.to_bits(w, "bf16")
    pw = bql.prepack_weight(dev16(bits, "bf16"), fmt)
    codes = host(bql.unpack_weight(pw))
    wf = oracle.decode_input(bits, "bf16")
    q, s = oracle.quant_per_tensor(wf) if fmt == "fp8_tensor" else oracle.quant_per_row(wf)
    s = np.atleast_1d(np.asarray(s, dtype=np.float32))
    got_s = host(pw.scales)
    assert np.array_equal(np.isnan(got_s), np.isnan(s))
    assert np.array_equal(got_s[~np.isnan(s)].view(np.uint32), s[~np.isnan(s)].view(np.uint32))
    nan = (q & 0x7F) == 0x7F
    assert nan.any() and np.array_equal((codes & 0x7F) == 0x7F, nan)
    assert np.array_equal(codes[~nan], q[~nan])


def test_prepack_given_fp16_channel_scales_w8a16_workload():
    N = K = 4096
    g = wl.rng(2, 0)
    bits = wl.weight(g, N, K, "f16")
    wf = oracle.decode_input(bits, "f16")
    sbits = wl.w8a16_channel_scales(g, wf)
    s32 = oracle.decode_input(sbits, "f16")
    pw = bql.prepack_weight(dev16(bits, "f16"), "fp8_channel", scales=dev16(sbits, "f16"))
    assert np.array_equal(host(pw.scales), s32)
    q = oracle.quant_with_scales(wf, s32)
    assert np.array_equal(host(bql.unpack_weight(pw)), q)
    sat = np.mean((q & 0x7F) == 0x7E)
    say(f"  saturated codes: {sat:.4%}")
    assert sat > 0  # about half the rows have a scale below amax/448


def test_prepack_e4m3_codes_pass_through():
    g = np.random.Generator(np.random.PCG64(21))
    N, K = 96, 400
    codes = g.integers(0, 256, (N, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    scales = g.uniform(0.5, 2, N).astype(np.float32)
    pw = bql.prepack_weight(dev(codes), "fp8_channel", scales=dev(scales))
    assert np.array_equal(host(bql.unpack_weight(pw)), codes)
    assert np.array_equal(host(pw.scales), scales)


@pytest.mark.parametrize("N,K", [(48, 144), (4096, 4096), (6656, 6656), (32, 16)])
def test_prepack_int4_round_trip(N, K):
    g = wl.rng(5, N, K, 1)
    w = wl.int4_weight(g, N, K)
    packed = wl.pack_int4(w)
    sbits = wl.w4a8_channel_scales(g, N)
    pw = bql.prepack_weight(dev(packed.reshape(N, K // 2)), "int4_channel", scales=dev16(sbits, "f16"))
    assert np.array_equal(host(bql.unpack_weight(pw)).ravel(), packed)
    assert np.array_equal(host(pw.scales), oracle.decode_input(sbits, "f16"))
