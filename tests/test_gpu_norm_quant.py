"""GPU parity of RMSNorm fused with the activation quantizers (QQQ issue #15:
the activation quantizer fused into an element-wise kernel such as rmsnorm)
against the CPU oracle.

The definition sums the squares in fp64 without fixing the order, so at a
row whose exact r lies next to an fp32 rounding boundary two fp32 values of
r are correct (oracle.rms_inv_candidates).  The GPU's r must be one of the
oracle's admissible values for its row; the oracle then quantizes with that
admissible value, and codes and scales must be identical bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import dev16, host, say

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu


def _inputs(seed, M, K, dtype, outliers):
    g = wl.rng(98, seed, M, K)
    xb = wl.activation(g, M, K, dtype, outliers)
    gb = wl.norm_weight(g, K, dtype)
    return xb, gb


def _pick_r(r_gpu, x, eps, what):
    lo, hi = oracle.rms_inv_candidates(x, eps)
    ok = (r_gpu == lo) | (r_gpu == hi)
    assert ok.all(), f"{what}: {int((~ok).sum())} rows with an inadmissible r"
    amb = int((lo != hi).sum())
    return np.where(r_gpu == lo, lo, hi), amb


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _run_int8(xb, gb, dtype, eps, what):
    M, K = xb.shape
    q, s, r = bql.rmsnorm_int8_quantize_per_token(dev16(xb, dtype), dev16(gb, dtype), eps,
                                                  inv_rms=True)
    torch.cuda.synchronize()
    x = oracle.decode_input(xb, dtype)
    gf = oracle.decode_input(gb, dtype)
    r_sel, amb = _pick_r(host(r), x, eps, what)
    q_ref, s_ref, _ = oracle.rmsnorm_int8_per_token(x, gf, eps, r=r_sel)
    assert np.array_equal(_bits(host(s)), _bits(s_ref)), f"{what}: scales differ"
    bad = np.nonzero(host(q).ravel() != q_ref.ravel())[0]
    assert bad.size == 0, f"{what}: {bad.size} codes differ, first at {bad[:5]}"
    say(f"  {what}: {M}x{K} int8 codes and scales identical ({amb} rows with two admissible r)")
    return q, s


def _run_fp8(xb, gb, dtype, eps, what):
    M, K = xb.shape
    q, s, r = bql.rmsnorm_fp8_quantize_dynamic(dev16(xb, dtype), dev16(gb, dtype), eps,
                                               inv_rms=True)
    torch.cuda.synchronize()
    x = oracle.decode_input(xb, dtype)
    gf = oracle.decode_input(gb, dtype)
    r_sel, amb = _pick_r(host(r), x, eps, what)
    q_ref, s_ref, _ = oracle.rmsnorm_fp8_per_tensor(x, gf, eps, r=r_sel)
    assert _bits(host(s))[0] == _bits(s_ref)[()], f"{what}: scale {host(s)[0]} vs {s_ref}"
    bad = np.nonzero(host(q).ravel() != q_ref.ravel())[0]
    assert bad.size == 0, f"{what}: {bad.size} codes differ, first at {bad[:5]}"
    say(f"  {what}: {M}x{K} E4M3 codes and scale identical ({amb} rows with two admissible r)")
    return q, s, q_ref, s_ref


# W4A8 activations (K = N in {4096, 5120, 6656, 8192}, fp16 N(0,1)), every M
W4A8_CASES = [(M, K) for K in wl.CFG5_KN for M in wl.CFG5_M]


@pytest.mark.parametrize("M,K", W4A8_CASES)
def test_rmsnorm_int8_w4a8_shapes(M, K):
    xb, gb = _inputs(1, M, K, "f16", "none")
    _run_int8(xb, gb, "f16", 1e-5, f"rmsnorm+int8 f16 M={M} K={K}")


# Llama-3-8B hidden (K = 4096) and Llama-70B hidden (K = 8192), bf16 with
# outlier channels, the inputs of the fp8 linears
FP8_CASES = [(M, 4096) for M in wl.CFG3_M] + [(M, 8192) for M in wl.CFG4_M]


@pytest.mark.parametrize("M,K", FP8_CASES)
def test_rmsnorm_fp8_llama_shapes(M, K):
    xb, gb = _inputs(2, M, K, "bf16", "channels")
    _run_fp8(xb, gb, "bf16", 1e-5, f"rmsnorm+fp8 bf16 M={M} K={K}")


# Both block sizes (256 threads up to K = 8192, 1024 above), minimal and
# ragged K, the largest K, both dtypes and several eps; more rows than the
# persistent grid has blocks (1024 of 256 threads, 512 of 1024), so that
# blocks walk several rows with their folds' LDS buffers alternating
EDGE_CASES = [(1, 16, "f16", 1e-6), (3, 48, "bf16", 1e-5), (5, 8192, "bf16", 1e-5),
              (7, 8208, "f16", 1e-5), (9, 14336, "bf16", 1e-5), (4, 28672, "f16", 1e-6),
              (2, 32768, "bf16", 1e-2), (33, 272, "f16", 0.5), (2500, 4096, "f16", 1e-5),
              (1100, 16384, "bf16", 1e-5)]


@pytest.mark.parametrize("M,K,dtype,eps", EDGE_CASES)
def test_rmsnorm_quant_edges(M, K, dtype, eps):
    xb, gb = _inputs(3, M, K, dtype, "entries")
    _run_int8(xb, gb, dtype, eps, f"rmsnorm+int8 {dtype} M={M} K={K} eps={eps}")
    _run_fp8(xb, gb, dtype, eps, f"rmsnorm+fp8 {dtype} M={M} K={K} eps={eps}")


def test_zero_and_extreme_rows():
    K = 1024
    xb, gb = _inputs(4, 6, K, "f16", "none")
    x = oracle.decode_input(xb, "f16")
    x[1] = 0.0                           # all-zero row: r = 1/sqrt(eps), y = 0
    x[2] = 0.0
    x[2, 5] = 65504.0                    # one huge entry
    x[3] *= np.float32(2.0 ** -20)       # f16 subnormals
    x[4, :] = np.float32(-3.0)           # constant row
    xb = wl.to_bits(x, "f16")
    _run_int8(xb, gb, "f16", 1e-5, "rmsnorm+int8 zero/huge/subnormal/constant rows")
    _run_fp8(xb, gb, "f16", 1e-5, "rmsnorm+fp8 zero/huge/subnormal/constant rows")
    # all rows zero: per-tensor scale 1, every code 0
    z = np.zeros((3, 64), dtype=np.uint16)
    q, s, _ = bql.rmsnorm_fp8_quantize_dynamic(dev16(z, "f16"), dev16(gb[:64], "f16"), 1e-5)
    assert host(s)[0] == np.float32(1.0) and not host(q).any()


def test_golden_rows_on_gpu():
    # the hand-derived rows of tests/golden/rmsnorm_worked.txt (K = 16):
    # x = [3, 4, 0...], eps = 1e-30 stands in for 0 (below every fp64
    # rounding of these sums, so r is the same fp32(0.8))
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, :2] = [3, 4]
    xb = wl.to_bits(x, "f16")
    gb = wl.to_bits(np.ones(16, dtype=np.float32), "f16")
    q, s, r = bql.rmsnorm_int8_quantize_per_token(dev16(xb, "f16"), dev16(gb, "f16"), 1e-30,
                                                  inv_rms=True)
    assert _bits(host(r))[0] == 0x3F4CCCCD
    assert _bits(host(s))[0] == 0x3CCE69A0 and list(host(q)[0, :2]) == [95, 127]
    q, s, _ = bql.rmsnorm_fp8_quantize_dynamic(dev16(xb, "f16"), dev16(gb, "f16"), 1e-30)
    assert _bits(host(s))[0] == 0x3BEA0EA1 and list(host(q)[0, :2]) == [0x7A, 0x7E]


def test_without_inv_rms_and_deterministic():
    xb, gb = _inputs(5, 64, 4096, "bf16", "channels")
    x, g = dev16(xb, "bf16"), dev16(gb, "bf16")
    a = bql.rmsnorm_int8_quantize_per_token(x, g, 1e-5)
    b = bql.rmsnorm_int8_quantize_per_token(x, g, 1e-5, inv_rms=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and a[2] is None
    c = bql.rmsnorm_fp8_quantize_dynamic(x, g, 1e-5)
    d = bql.rmsnorm_fp8_quantize_dynamic(x, g, 1e-5, inv_rms=True)
    assert torch.equal(c[0], d[0]) and torch.equal(c[1], d[1])


def test_fused_fp8_codes_feed_the_linear():
    # RMSNorm + E4M3 codes go straight into the pre-quantized fp8 linear
    M, N, K = 128, 1024, 4096
    xb, gb = _inputs(6, M, K, "bf16", "channels")
    q, s, q_ref, s_ref = _run_fp8(xb, gb, "bf16", 1e-5, "rmsnorm+fp8 ahead of the linear")
    gw = wl.rng(98, 7)
    wb = wl.weight(gw, N, K, "bf16")
    pw = bql.prepack_weight(dev16(wb, "bf16"), "fp8_tensor")
    y = bql.fp8_linear(q, pw, a_scale=s, out_dtype=torch.float32)
    torch.cuda.synchronize()
    wq, sw = oracle.quant_per_tensor(oracle.decode_input(wb, "bf16"))
    ref = oracle.fp8_linear(q_ref, s_ref, wq, sw)
    ok, worst = oracle.within_tolerance(host(y).astype(np.float64), ref)
    assert ok, f"linear after rmsnorm+fp8: worst {worst}"
    say(f"  linear on rmsnorm+fp8 codes: worst |d|/bound = {worst:.3g}")
