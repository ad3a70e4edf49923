"""GPU parity of the per-group W4A8 linear (QQQ issue #15, the "qqq-g128"
columns: one scale per output channel and group of 128 k) against the CPU
oracle.

Float outputs within the stated tolerance over the W4A8 workload's shapes
(K = N in {4096, 5120, 6656, 8192}, M in {1, 16, 256, 1024}) and ragged
shapes; bit-exact where every fp32 partial sum is exact (small integers,
power-of-two scales), which checks that each group's scale lands on its own
channel and k range; the prepacked group scales equal the given ones.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import DEV, assert_close, dev, dev16, host, host_f64, rows_for, say

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu


def _pack(w4, sw_bits_or_f32, K):
    N = w4.shape[0]
    wpk = torch.from_numpy(wl.pack_int4(w4).reshape(N, K // 2)).to(DEV)
    if sw_bits_or_f32.dtype == np.uint16:
        sc = torch.from_numpy(sw_bits_or_f32.view(np.int16)).to(DEV).view(torch.float16)
    else:
        sc = dev(sw_bits_or_f32)
    return bql.prepack_weight(wpk, "int4_group", scales=sc)


def _group_scales(g, N, G):
    s = g.uniform(0.5, 2.0, size=(N, G)).astype(np.float32) * np.float32(2.0 ** -8)
    return wl.f32_to_f16_bits(s)


@pytest.mark.parametrize("M", wl.CFG5_M)
@pytest.mark.parametrize("KN", wl.CFG5_KN)
def test_w4a8_group_workload(M, KN):
    N = K = KN
    g = wl.rng(95, KN, M)
    w4 = wl.int4_weight(g, N, K)
    sbits = _group_scales(g, N, K // 128)
    pw = _pack(w4, sbits, K)
    sw = oracle.decode_input(sbits, "f16")
    assert np.array_equal(host(pw.scales).reshape(K // 128, N), sw.T), "group scales differ"
    ab = wl.activation(g, M, K, "f16")
    aq, sa = oracle.int8_quant_per_token(oracle.decode_input(ab, "f16"))
    y = bql.w4a8_group_linear(dev(aq), dev(sa), pw, out_dtype=torch.float16)
    torch.cuda.synchronize()
    rows = rows_for(M, 400 + M, 24)
    ref = oracle.w4a8_group_linear(aq, sa, w4, sw, rows=rows)
    assert_close(host_f64(y)[rows], ref, f"W4A8 g128 M={M} K=N={KN}")


@pytest.mark.parametrize("M,N,K", [(77, 1040, 384), (3, 16, 128), (300, 272, 1280), (16, 2064, 4096)])
@pytest.mark.parametrize("out", [torch.float16, torch.bfloat16, torch.float32])
def test_w4a8_group_ragged(M, N, K, out):
    g = wl.rng(95, M, N, K)
    w4 = wl.int4_weight(g, N, K)
    sw = (g.uniform(0.5, 2.0, size=(N, K // 128)) * 2.0 ** -8).astype(np.float32)
    pw = _pack(w4, sw, K)
    aq = g.integers(-127, 128, size=(M, K), dtype=np.int8)
    sa = g.uniform(1e-3, 1e-1, size=M).astype(np.float32)
    y = bql.w4a8_group_linear(dev(aq), dev(sa), pw, out_dtype=out)
    torch.cuda.synchronize()
    assert_close(host_f64(y), oracle.w4a8_group_linear(aq, sa, w4, sw), f"g128 M={M} N={N} K={K} {out}")


@pytest.mark.parametrize("M", [1, 8, 512])
def test_w4a8_group_exact_small_integers(M):
    # every partial sum is an integer below 2^24 and every scale a power of
    # two, so the fp32 result is exact: it must equal the oracle bit for bit
    N, K = 256, 2048
    g = np.random.Generator(np.random.PCG64(M))
    w4 = g.integers(-2, 3, size=(N, K), dtype=np.int8)
    aq = g.integers(-3, 4, size=(M, K), dtype=np.int8)
    sw = (2.0 ** g.integers(-6, 3, size=(N, K // 128))).astype(np.float32)
    sa = (2.0 ** g.integers(-4, 2, size=M)).astype(np.float32)
    pw = _pack(w4, sw, K)
    y = bql.w4a8_group_linear(dev(aq), dev(sa), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.w4a8_group_linear(aq, sa, w4, sw)
    assert np.array_equal(host(y).astype(np.float64), ref), "per-group result not exact"
    say(f"  M={M}: per-group W4A8 bit-exact on exact inputs")


def test_w4a8_group_unpack_roundtrip():
    N, K = 64, 512
    w4 = wl.int4_weight(wl.rng(95, 1), N, K)
    pw = _pack(w4, np.ones((N, K // 128), np.float32), K)
    assert np.array_equal(host(bql.unpack_weight(pw)).ravel(), wl.pack_int4(w4))
