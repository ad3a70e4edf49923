"""GPU parity of the activation quantizers against the CPU oracle (bit-exact).

Dynamic per-tensor E4M3 (vLLM PR #4118, "Algorithm") and the per-token int8
quantizer of the W4A8 path (QQQ issue #15).  Codes and scales must be
identical to the oracle's, byte for byte.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import DEV, dev16, host, say

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_dynamic(bits: np.ndarray, dtype: str, what: str):
    x = dev16(bits, dtype)
    xq, s = bql.quantize_dynamic(x)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_per_tensor(oracle.decode_input(bits, dtype))
    got_s = host(s)[0]
    assert got_s.view(np.uint32) == np.float32(s_ref).view(np.uint32), f"{what}: scale {got_s} vs {s_ref}"
    got = host(xq)
    bad = np.nonzero(got.ravel() != q_ref.ravel())[0]
    assert bad.size == 0, f"{what}: {bad.size} codes differ, first at {bad[:5]}"
    say(f"  {what}: {bits.size} codes identical, scale {s_ref!r}")


def test_worked_example():
    x = wl.to_bits(np.array([1.0, -3.5, 0.1, 7.0], dtype=np.float32), "f16")
    xq, s = bql.quantize_dynamic(dev16(x, "f16"))
    assert host(s)[0] == np.float32(2.0 ** -6)
    assert list(host(xq)) == [0x68, 0xF6, 0x4D, 0x7E]


def _finite_patterns(dtype):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if dtype == "f16":
        return b[((b >> 10) & 31) != 31]
    return b[((b >> 7) & 255) != 255]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_exhaustive_patterns_dynamic(dtype):
    _check_dynamic(_finite_patterns(dtype), dtype, f"all finite {dtype} patterns, dynamic")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.0123, 2.0 ** -6, 37.5, 1e-3, 300.0, 3.0e-7])
def test_exhaustive_patterns_static(dtype, scale):
    bits = _finite_patterns(dtype)
    s = np.float32(scale)
    xq = bql.quantize_static(dev16(bits, dtype), torch.tensor([s], device=DEV))
    q_ref = oracle.quant_with_scales(oracle.decode_input(bits, dtype).reshape(1, -1), np.array([s]))
    got = host(xq)
    bad = np.nonzero(got != q_ref.ravel())[0]
    assert bad.size == 0, f"{bad.size} codes differ, e.g. bits {bits[bad[:4]]} got {got[bad[:4]]} want {q_ref.ravel()[bad[:4]]}"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.0123])
def test_static_nonfinite_inputs(dtype, scale):
    """Every infinity and NaN pattern, plus signed zeros, with a caller's
    scale: infinities saturate to the +-448 codes and NaNs give the NaN codes
    with their sign kept, as the oracle encodes them."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    nonfinite = b[((b >> 10) & 31) == 31] if dtype == "f16" else b[((b >> 7) & 255) == 255]
    bits = np.concatenate([nonfinite, np.array([0x0000, 0x8000], dtype=np.uint16)])
    s = np.float32(scale)
    xq = bql.quantize_static(dev16(bits, dtype), torch.tensor([s], device=DEV))
    q_ref = oracle.quant_with_scales(oracle.decode_input(bits, dtype).reshape(1, -1), np.array([s])).ravel()
    got = host(xq)
    assert set(np.unique(q_ref).tolist()) == {0x00, 0x80, 0x7E, 0xFE, 0x7F, 0xFF}
    bad = np.nonzero(got != q_ref)[0]
    assert bad.size == 0, f"{bad.size} codes differ, e.g. bits {bits[bad[:4]]} got {got[bad[:4]]} want {q_ref[bad[:4]]}"


@pytest.mark.parametrize("M,K", [(16, 1024), (1, 4096), (16, 14336), (128, 4096), (1024, 14336),
                                 (1024, 4096)])
def test_config_activations(M, K):
    dtype = "f16" if K == 1024 else "bf16"
    cfg = 1 if K == 1024 else 3
    g = wl.rng(cfg, M, K, 2)
    bits = wl.activation(g, M, K, dtype, "entries" if cfg == 1 else "channels")
    _check_dynamic(bits, dtype, f"cfg{cfg} A {M}x{K} {dtype}")


@pytest.mark.parametrize("n", [1, 7, 8, 9, 4095, 1000003])
def test_ragged_lengths(n):
    g = wl.rng(9, n)
    bits = wl.activation(g, 1, n, "bf16", "entries")
    _check_dynamic(bits.ravel(), "bf16", f"ragged n={n}")


def test_amax_in_the_ragged_tail_and_zero_tensor():
    bits = np.zeros(1000005, dtype=np.uint16)
    _check_dynamic(bits, "f16", "all zeros")
    x = np.zeros(1000005, dtype=np.float32)
    x[-1] = -1234.5
    x[5] = 3.0
    _check_dynamic(wl.to_bits(x, "bf16"), "bf16", "amax in the tail")


# ------------------------------------------------------------- int8 per token

@pytest.mark.parametrize("M,K", [(1, 4096), (16, 5120), (256, 6656), (1024, 8192), (3, 48)])
def test_int8_per_token(M, K):
    g = wl.rng(5, M, K, 2)
    bits = wl.activation(g, M, K, "f16")
    if M >= 3:
        bits[1] = 0  # an all-zero row takes scale 1
    q, s = bql.int8_quantize_per_token(dev16(bits, "f16"))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.int8_quant_per_token(oracle.decode_input(bits, "f16"))
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(q), q_ref)
    say(f"  int8 per-token {M}x{K}: identical")


def test_int8_worked_rows():
    x = np.array([[127, -63.5, 0.5, 1.5] * 4, [-254, 1, 3, 5] * 4], dtype=np.float32)
    q, s = bql.int8_quantize_per_token(dev16(wl.to_bits(x, "f16"), "f16"))
    assert list(host(s)) == [1.0, 2.0]
    assert list(host(q)[0][:4]) == [127, -64, 0, 2]
    assert list(host(q)[1][:4]) == [-127, 0, 2, 2]


@pytest.mark.parametrize("n", [4096, 1000005])
@pytest.mark.parametrize("kind", ["nan", "inf"])
def test_dynamic_nonfinite_tensor(n, kind):
    """A NaN anywhere makes the amax, the scale and every code NaN; an
    infinity makes the scale infinite, every finite value a zero code of its
    sign and the infinity itself the NaN code.  The sign of a NaN made by a
    division is not fixed by IEEE 754, so NaN codes may carry either sign."""
    g = wl.rng(10, n)
    x = oracle.decode_input(wl.activation(g, 1, n, "bf16", "channels"), "bf16").ravel().astype(np.float32)
    x[n // 3] = np.nan if kind == "nan" else np.inf
    bits = wl.to_bits(x, "bf16")
    xq, s = bql.quantize_dynamic(dev16(bits, "bf16"))
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):
        q_ref, s_ref = oracle.quant_per_tensor(oracle.decode_input(bits, "bf16"))
    got_s = host(s)[0]
    assert (np.isnan(got_s) and np.isnan(s_ref)) or got_s == s_ref
    got = host(xq)
    nan = (q_ref & 0x7F) == 0x7F
    assert np.array_equal((got & 0x7F) == 0x7F, nan)
    assert np.array_equal(got[~nan], q_ref[~nan])

