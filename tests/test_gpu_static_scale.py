"""GPU parity of the fp8 linear with a static activation scale (vLLM
discussion #5802, "RFC: FP8 Quantization Schema": per-tensor static scaling
with the input_scale from the checkpoint; also a delayed scale kept from an
earlier call) against the CPU oracle.

Aq = E4M3(fp32(A / a_scale)) with the given scale, no amax pass; the linear
is then the one of vLLM PR #4118.  Checks: with the dynamic scale as the
static one, outputs are bitwise those of the dynamic call on every path
(fused small-M, small-M, tiled; both accumulation modes); codes are
bit-exact against the oracle for arbitrary scales (a one-hot weight makes
Y = sA * dec(Aq) exactly); float outputs within the stated tolerance for
scales that leave A unsaturated or saturate much of it.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import DEV, Weights, assert_close, dev, dev16, host, host_f64, rows_for, say

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def _weights(idx, N, K, dtype, per_channel):
    W = Weights(3, idx, N, K, dtype, per_channel)
    pw = bql.prepack_weight(dev16(W.bits, dtype), "fp8_channel" if per_channel else "fp8_tensor")
    return W, pw


def _act(M, K, dtype, seed):
    return wl.activation(wl.rng(97, seed, M, K), M, K, dtype, "channels")


# fused small-M (M <= 4, and M = 16 at K = 1024), small-M with A quantized
# by its own launch (M = 16, K = 4096 and 14336), tiled (M = 77, 128, 1024)
EQUIV = [(1, 4096, 4096), (4, 6144, 4096), (16, 1024, 1024), (16, 6144, 4096),
         (16, 4096, 14336), (128, 4096, 4096), (1024, 6144, 4096), (3, 1024, 1024),
         (77, 1040, 528)]


@pytest.mark.parametrize("M,N,K", EQUIV)
@pytest.mark.parametrize("fast", [False, True])
def test_dynamic_scale_as_static_is_bitwise_the_dynamic_call(M, N, K, fast):
    W, pw = _weights(0, N, K, "bf16", False)
    a = dev16(_act(M, K, "bf16", 1), "bf16")
    sa = torch.empty(1, dtype=torch.float32, device=DEV)
    y_dyn = bql.fp8_linear(a, pw, a_scale=sa, out_dtype=torch.bfloat16, fast_accum=fast)
    y_st = bql.fp8_linear_static(a, pw, sa, out_dtype=torch.bfloat16, fast_accum=fast)
    torch.cuda.synchronize()
    assert torch.equal(y_dyn.view(torch.int16), y_st.view(torch.int16)), f"M={M} N={N} K={K}"
    say(f"  M={M} N={N} K={K} fast={fast}: static == dynamic, bitwise")


def _one_hot_weight(K):
    """E4M3 codes of the identity [K, K] (1.0 = 0x38) with scale 1."""
    codes = np.zeros((K, K), dtype=np.uint8)
    codes[np.arange(K), np.arange(K)] = 0x38
    pw = bql.prepack_weight(dev(codes), "fp8_tensor",
                            scales=torch.tensor([1.0], dtype=torch.float32, device=DEV))
    return pw


def _all_finite_f16(count, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    b = g.integers(0, 65536, size=count * 2, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 10) & 31) != 31]
    return b[:count]


@pytest.mark.parametrize("M", [1, 4, 16, 128])
@pytest.mark.parametrize("scale", [2.0 ** -6, 0.0123, 37.5, 3.0e-7, 1.0e-3, 300.0])
def test_static_codes_bit_exact(M, scale):
    K = 256
    pw = _one_hot_weight(K)
    bits = _all_finite_f16(M * K, int(scale * 1e9) % 1000 + M).reshape(M, K)
    s = np.float32(scale)
    y = bql.fp8_linear_static(dev16(bits, "f16"), pw, torch.tensor([s], device=DEV),
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    q_ref = oracle.quant_with_scales(oracle.decode_input(bits, "f16"), np.array([s], np.float32))
    tab = oracle.e4m3_decode_table()
    ref = (np.float32(s) * tab[q_ref.astype(np.int64)].astype(np.float32)).astype(np.float32)
    got = host(y)
    same = (got == ref) | ((got == 0) & (ref == 0))  # the sign of a zero sum is not kept
    assert same.all(), f"M={M} s={scale}: {int((~same).sum())} codes differ"
    say(f"  M={M} scale={scale}: {M * K} codes identical")


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (16, 6144, 4096), (128, 28672, 4096),
                                   (1024, 4096, 14336)])
@pytest.mark.parametrize("mult", [2.0, 0.25])
def test_static_scale_vs_oracle(M, N, K, mult):
    W, pw = _weights(wl.CFG3_SHAPES.index((N, K)), N, K, "bf16", True)
    bits = _act(M, K, "bf16", 2)
    x = oracle.decode_input(bits, "bf16")
    # a calibrated scale: mult * amax / 448 (0.25 saturates much of A)
    s = np.float32(np.float32(np.abs(x).max()) / np.float32(448.0) * np.float32(mult))
    y = bql.fp8_linear_static(dev16(bits, "bf16"), pw, torch.tensor([s], device=DEV),
                              out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = rows_for(M, 200 + M, 24)
    aq = oracle.quant_with_scales(x[rows], np.array([s], np.float32))
    y_ref = oracle.fp8_linear(aq, s, W.codes, W.scales)
    assert_close(host_f64(y)[rows], y_ref, f"static M={M} N={N} K={K} scale x{mult}")


def test_delayed_scale_from_an_earlier_call():
    # the scale of one call's activations reused for the next call's
    M, N, K = 64, 4096, 4096
    W, pw = _weights(1, N, K, "bf16", False)
    b1, b2 = _act(M, K, "bf16", 3), _act(M, K, "bf16", 4)
    sa = torch.empty(1, dtype=torch.float32, device=DEV)
    bql.fp8_linear(dev16(b1, "bf16"), pw, a_scale=sa, out_dtype=torch.bfloat16)
    y = bql.fp8_linear_static(dev16(b2, "bf16"), pw, sa, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _, s1 = oracle.quant_per_tensor(oracle.decode_input(b1, "bf16"))
    assert host(sa)[0] == s1
    aq = oracle.quant_with_scales(oracle.decode_input(b2, "bf16"), np.array([s1], np.float32))
    y_ref = oracle.fp8_linear(aq, s1, W.codes, W.scales)
    assert_close(host_f64(y), y_ref, "delayed scale")


def test_static_fp8_output():
    M, N, K = 128, 4096, 4096
    W, pw = _weights(1, N, K, "bf16", False)
    bits = _act(M, K, "bf16", 5)
    x = oracle.decode_input(bits, "bf16")
    s = np.float32(np.float32(np.abs(x).max()) / np.float32(448.0))
    aq = oracle.quant_with_scales(x, np.array([s], np.float32))
    y_ref = oracle.fp8_linear(aq, s, W.codes, W.scales)
    osc = np.float32(np.abs(y_ref).max() / 448.0)
    yq = bql.fp8_linear_static(dev16(bits, "bf16"), pw, torch.tensor([s], device=DEV),
                               out_dtype=torch.float8_e4m3fn,
                               output_scale=torch.tensor([osc], device=DEV))
    torch.cuda.synchronize()
    from _common import assert_fp8_out
    assert_fp8_out(host(yq), y_ref / np.float64(osc), "static scale, fp8 out")
