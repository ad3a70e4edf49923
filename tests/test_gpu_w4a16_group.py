"""GPU parity of the per-group weight-only int4 linear (QQQ issue #15, the
"awq-g128" and "marlin-g128" columns: fp16 activations, int4 weights, one
scale per output channel and group of 128 k) against the CPU oracle.

Float outputs within the stated tolerance over the W4A8 workload's shapes
(K = N in {4096, 5120, 6656, 8192}, M in {1, 16, 256, 1024}, the same
models' weight-only rows of the tables) and ragged shapes; bit-exact where
every fp32 partial sum is exact (small integers, power-of-two scales), which
checks the int4 -> fp16 decode of every nibble position and that each
group's scale lands on its own channel and k range.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import DEV, assert_close, dev, dev16, host, host_f64, rows_for, say

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu


def _pack(w4, sw, K):
    N = w4.shape[0]
    wpk = torch.from_numpy(wl.pack_int4(w4).reshape(N, K // 2)).to(DEV)
    if sw.dtype == np.uint16:
        sc = torch.from_numpy(sw.view(np.int16)).to(DEV).view(torch.float16)
    else:
        sc = dev(sw)
    return bql.prepack_weight(wpk, "int4_group", scales=sc)


@pytest.mark.parametrize("M", wl.CFG5_M)
@pytest.mark.parametrize("KN", wl.CFG5_KN)
def test_w4a16_group_workload(M, KN):
    N = K = KN
    g = wl.rng(94, KN, M)
    w4 = wl.int4_weight(g, N, K)
    sbits = wl.f32_to_f16_bits(g.uniform(0.5, 2.0, size=(N, K // 128)).astype(np.float32)
                               * np.float32(2.0 ** -8))
    pw = _pack(w4, sbits, K)
    sw = oracle.decode_input(sbits, "f16")
    ab = wl.activation(g, M, K, "f16")
    y = bql.w4a16_group_linear(dev16(ab, "f16"), pw, out_dtype=torch.float16)
    torch.cuda.synchronize()
    rows = rows_for(M, 500 + M, 24)
    ref = oracle.w4a16_group_linear(oracle.decode_input(ab, "f16").reshape(M, K), w4, sw, rows=rows)
    assert_close(host_f64(y)[rows], ref, f"W4A16 g128 M={M} K=N={KN}")


# M above 16 runs the tile kernel (128 x 256 blocks): partial row blocks
# (77, 300, 130), a column block with waves wholly past N (272), one and
# two k-tiles (the pipeline's shortest runs), odd k-tile counts (384), and
# few blocks with a long K, whose k range is split over blocks (fp32
# partial sums, then the split-K reduce): (200, 1040, 4096); blocks of 128
# columns at most of these shapes and 256 columns where 128 would take a
# second round: (2000, 2064, 1024) unsplit, (520, 4208, 4096) in three K
# splits; (8, 256, 65536): the small-M kernel with K split eight ways
@pytest.mark.parametrize("M,N,K", [(77, 1040, 384), (3, 16, 128), (300, 272, 1280), (16, 2064, 4096),
                                   (1, 4096, 14336), (40, 512, 128), (130, 4096, 256), (17, 784, 640),
                                   (200, 1040, 4096), (1024, 4096, 4096), (8, 256, 65536),
                                   (2000, 2064, 1024), (520, 4208, 4096)])
@pytest.mark.parametrize("out", [torch.float16, torch.bfloat16, torch.float32])
def test_w4a16_group_ragged(M, N, K, out):
    g = wl.rng(94, M, N, K)
    w4 = wl.int4_weight(g, N, K)
    sw = (g.uniform(0.5, 2.0, size=(N, K // 128)) * 2.0 ** -8).astype(np.float32)
    pw = _pack(w4, sw, K)
    ab = wl.activation(g, M, K, "f16", "entries")  # outlier entries x20
    y = bql.w4a16_group_linear(dev16(ab, "f16"), pw, out_dtype=out)
    torch.cuda.synchronize()
    ref = oracle.w4a16_group_linear(oracle.decode_input(ab, "f16").reshape(M, K), w4, sw)
    assert_close(host_f64(y), ref, f"W4A16 g128 M={M} N={N} K={K} {out}")


@pytest.mark.parametrize("M", [1, 8, 40, 300])
def test_w4a16_group_exact_small_integers(M):
    # every nibble value -8..7 in every byte position, integer activations
    # and power-of-two group scales: all fp32 partial sums are exact, so the
    # result must equal the oracle bit for bit
    N, K = 256, 2048
    g = np.random.Generator(np.random.PCG64(40 + M))
    w4 = g.integers(-8, 8, size=(N, K), dtype=np.int8)
    a = g.integers(-2, 3, size=(M, K)).astype(np.float32)  # |acc| < 2^17 in steps of 2^-6
    sw = (2.0 ** g.integers(-6, 3, size=(N, K // 128))).astype(np.float32)
    pw = _pack(w4, sw, K)
    y = bql.w4a16_group_linear(dev(a.astype(np.float16)), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.w4a16_group_linear(a, w4, sw)
    assert np.array_equal(host(y).astype(np.float64), ref), "per-group W4A16 result not exact"
    say(f"  M={M}: per-group W4A16 bit-exact on exact inputs")


def test_w4a16_group_each_nibble_position():
    # a one-hot activation reads out one weight column: every (channel, k)
    # int4 value through the decode, times its group's scale, exactly
    N, K = 32, 256
    g = np.random.Generator(np.random.PCG64(7))
    w4 = g.integers(-8, 8, size=(N, K), dtype=np.int8)
    sw = (2.0 ** g.integers(-3, 3, size=(N, K // 128))).astype(np.float32)
    pw = _pack(w4, sw, K)
    a = np.eye(K, dtype=np.float16)          # M = K rows, row k picks k
    y = host(bql.w4a16_group_linear(dev(a), pw, out_dtype=torch.float32))
    torch.cuda.synchronize()
    expect = (w4.astype(np.float32) * np.repeat(sw, 128, axis=1)).T  # [K, N]
    assert np.array_equal(y, expect)
