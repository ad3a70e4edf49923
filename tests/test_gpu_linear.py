"""GPU parity of the linears against the CPU oracle.

fp8 linear Y = (sA sW[n]) (Aq Wq^T) with dynamic per-tensor activation
scaling (vLLM PR #4118), per-tensor or per-channel weight scales
(optimum-quanto PR #241), fp16/bf16 output or fp8 output with an
output_scale (vLLM discussion #5802); W8A16 (optimum-quanto PR #241);
W4A8 with int32 accumulation (QQQ issue #15).

Float outputs: |d| <= 5e-3 (|ref| + 1e-2 max|ref|).  Activation scales and
int32 accumulators: identical.  Large outputs are checked on seeded sampled
rows (first and last included), computed one by one by the oracle.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import (DEV, TORCH_DT, Weights, assert_close, assert_fast_bound, assert_fp8_out, dev,
                     dev16, host, host_f64, rows_for, say)

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def _weights(cfg, idx, N, K, dtype, per_channel):
    return Weights(cfg, idx, N, K, dtype, per_channel)


@functools.lru_cache(maxsize=2)
def _packed(cfg, idx, N, K, dtype, per_channel):
    W = _weights(cfg, idx, N, K, dtype, per_channel)
    pw = bql.prepack_weight(dev16(W.bits, dtype), "fp8_channel" if per_channel else "fp8_tensor")
    assert np.array_equal(host(pw.scales).view(np.uint32), W.scales.view(np.uint32))
    return pw


def _fp8_case(cfg, idx, M, N, K, dtype, per_channel, outliers, out_dtype, rows_count=32,
              fp8_out=False):
    W = _weights(cfg, idx, N, K, dtype, per_channel)
    pw = _packed(cfg, idx, N, K, dtype, per_channel)
    g = wl.rng(cfg, idx, M, 3)
    a_bits = wl.activation(g, M, K, dtype, outliers)
    a = dev16(a_bits, dtype)
    a_scale = torch.empty(1, dtype=torch.float32, device=DEV)
    y = bql.fp8_linear(a, pw, a_scale=a_scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    aq_ref, sa_ref = oracle.quant_per_tensor(oracle.decode_input(a_bits, dtype))
    assert host(a_scale)[0].view(np.uint32) == np.float32(sa_ref).view(np.uint32)
    rows = rows_for(M, 100 + M, rows_count)
    y_ref = oracle.fp8_linear(aq_ref, sa_ref, W.codes, W.scales, rows=rows)
    assert_close(host_f64(y)[rows], y_ref, f"cfg{cfg} M={M} N={N} K={K} {out_dtype}")
    # the fp8 matrix cores' own accumulation, against its derived bound
    yf = bql.fp8_linear(a, pw, out_dtype=out_dtype, fast_accum=True)
    torch.cuda.synchronize()
    sw = W.scales if W.scales.size == N else np.full(N, W.scales[0], dtype=np.float32)
    abs_sum = oracle.fp8_acc(aq_ref & 0x7F, W.codes & 0x7F, rows=rows) * np.float64(sa_ref) \
        * sw.astype(np.float64)[None, :]
    assert_fast_bound(host_f64(yf)[rows], y_ref, abs_sum, f"cfg{cfg} M={M} fast accumulation")
    if fp8_out:
        for mult in (1.0, 0.5):  # 0.5: part of the output saturates
            osc = np.float32(np.abs(y_ref).max() / 448.0 * mult)
            yq = bql.fp8_linear(a, pw, out_dtype=torch.float8_e4m3fn,
                                output_scale=torch.tensor([osc], device=DEV))
            torch.cuda.synchronize()
            assert_fp8_out(host(yq)[rows], y_ref / np.float64(osc), f"  fp8 out x{mult}")
    return y


# -------------------------------------------------------------- config 1

def test_cfg1_w8a8_small():
    _fp8_case(1, 0, 16, 1024, 1024, "f16", False, "entries", torch.float16)


# -------------------------------------------------------------- config 3

@pytest.mark.parametrize("idx", range(4))
@pytest.mark.parametrize("M", wl.CFG3_M)
def test_cfg3_llama3_8b(idx, M):
    N, K = wl.CFG3_SHAPES[idx]
    _fp8_case(3, idx, M, N, K, "bf16", False, "channels", torch.bfloat16)


@pytest.mark.parametrize("K", [256, 1200])
@pytest.mark.parametrize("M", [1, 3, 16])
def test_small_m_two_strip_blocks_odd_count(M, K):
    """N = 16400: 1025 channel strips, above the count where the small-M fp8
    kernel gives each block two strips, so the last block has one; dynamic
    quantization (fused into the GEMV for M <= 4 and, at K = 256, M = 16),
    then pre-quantized A (row-major).  The fused two-strip blocks request
    two k-tiles per wave before the prologue: K = 256 leaves six of the
    eight waves without a k-tile, K = 1200 (ten k-tiles, the last ragged)
    gives two waves a second one."""
    _fp8_case(3, 7 if K == 256 else 8, M, 16400, K, "bf16", False, "channels", torch.bfloat16)
    g = np.random.Generator(np.random.PCG64(54 + M + K))
    N = 16400
    aq = _random_codes(g, (M, K))
    wq = _random_codes(g, (N, K))
    sa, sw = np.float32(0.5), np.float32(0.25)
    pw = bql.prepack_weight(dev(wq), "fp8_tensor", scales=torch.tensor([sw], device=DEV))
    y_ref = oracle.fp8_linear(aq, sa, wq, np.array([sw], dtype=np.float32))
    for fast in (False, True):
        y = bql.fp8_linear(dev(aq).view(torch.float8_e4m3fn), pw, a_scale=torch.tensor([sa], device=DEV),
                           out_dtype=torch.float32, fast_accum=fast)
        torch.cuda.synchronize()
        if fast:
            abs_sum = oracle.fp8_acc(aq & 0x7F, wq & 0x7F) * np.float64(sa) * np.float64(sw)
            assert_fast_bound(host_f64(y), y_ref, abs_sum, f"pre-quantized M={M} N={N} fast")
        else:
            assert_close(host_f64(y), y_ref, f"pre-quantized M={M} N={N}")


# -------------------------------------------------------------- config 4

@pytest.mark.parametrize("idx", range(4))
@pytest.mark.parametrize("M", wl.CFG4_M)
def test_cfg4_llama70b_prefill(idx, M):
    N, K = wl.CFG4_SHAPES[idx]
    _fp8_case(4, idx, M, N, K, "bf16", True, "channels", torch.bfloat16, rows_count=16,
              fp8_out=True)


# -------------------------------------------------------------- config 2

@pytest.mark.parametrize("M", [1, 8])
def test_cfg2_w8a16_decode(M):
    N = K = 4096
    g = wl.rng(2, 0)
    bits = wl.weight(g, N, K, "f16")
    wf = oracle.decode_input(bits, "f16")
    sbits = wl.w8a16_channel_scales(g, wf)
    s32 = oracle.decode_input(sbits, "f16")
    codes = oracle.quant_with_scales(wf, s32)
    pw = bql.prepack_weight(dev16(bits, "f16"), "fp8_channel", scales=dev16(sbits, "f16"))
    a_bits = wl.activation(wl.rng(2, M, 3), M, K, "f16")
    y = bql.w8a16_linear(dev16(a_bits, "f16"), pw, out_dtype=torch.float16)
    torch.cuda.synchronize()
    y_ref = oracle.w8a16_linear(oracle.decode_input(a_bits, "f16"), codes, s32)
    assert_close(host_f64(y), y_ref, f"cfg2 W8A16 M={M}")


# -------------------------------------------------------------- config 5

@functools.lru_cache(maxsize=1)
def _int4(idx, N, K):
    g = wl.rng(5, idx, 1)
    w = wl.int4_weight(g, N, K)
    sbits = wl.w4a8_channel_scales(g, N)
    pw = bql.prepack_weight(dev(wl.pack_int4(w).reshape(N, K // 2)), "int4_channel",
                            scales=dev16(sbits, "f16"))
    return w, oracle.decode_input(sbits, "f16"), pw


@pytest.mark.parametrize("idx", range(4))
@pytest.mark.parametrize("M", wl.CFG5_M)
def test_cfg5_w4a8(idx, M):
    N = K = wl.CFG5_KN[idx]
    w, sw, pw = _int4(idx, N, K)
    a_bits = wl.activation(wl.rng(5, idx, M, 3), M, K, "f16")
    aq, sa = bql.int8_quantize_per_token(dev16(a_bits, "f16"))
    acc = bql.w4a8_linear(aq, sa, pw, out_dtype=torch.int32)
    y = bql.w4a8_linear(aq, sa, pw, out_dtype=torch.float16)
    torch.cuda.synchronize()
    aq_ref, sa_ref = oracle.int8_quant_per_token(oracle.decode_input(a_bits, "f16"))
    assert np.array_equal(host(aq), aq_ref) and np.array_equal(host(sa), sa_ref)
    rows = rows_for(M, 500 + M, 64)
    acc_ref = oracle.w4a8_acc(aq_ref, w, rows=rows)
    got = host(acc)[rows].astype(np.int64)
    assert np.array_equal(got, acc_ref), f"int32 accumulators differ at {np.argwhere(got != acc_ref)[:4]}"
    assert_close(host_f64(y)[rows], oracle.w4a8_linear(acc_ref, sa_ref, sw, rows=rows),
                 f"cfg5 W4A8 M={M} N=K={N}")


# ---------------------------------------------------------- edge cases

# M = 16 / 17: the small-M kernel / the tile kernels; 128 / 129: the
# k-split kernel / the exact 256-row kernel
@pytest.mark.parametrize("M", [1, 3, 16, 17, 128, 129, 130, 300])
@pytest.mark.parametrize("N,K", [(48, 144), (16, 16), (272, 400)])
def test_fp8_ragged(M, N, K):
    _fp8_case(8, N * 1000 + K, M, N, K, "bf16", True, "entries", torch.bfloat16, rows_count=400)


# W8A16 streams the weight once per 16-row batch at every M
@pytest.mark.parametrize("M", [1, 5, 16, 17, 40, 129])
@pytest.mark.parametrize("N,K", [(48, 144), (272, 400)])
def test_w8a16_ragged(M, N, K):
    g = wl.rng(9, N, K)
    bits = wl.weight(g, N, K, "f16")
    pw = bql.prepack_weight(dev16(bits, "f16"), "fp8_channel")
    codes, s = oracle.quant_per_row(oracle.decode_input(bits, "f16"))
    a_bits = wl.activation(wl.rng(9, M), M, K, "f16")
    y = bql.w8a16_linear(dev16(a_bits, "f16"), pw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_close(host_f64(y), oracle.w8a16_linear(oracle.decode_input(a_bits, "f16"), codes, s),
                 f"W8A16 M={M} N={N} K={K}")


# M = 16 / 17: the small-M kernel / the 128 x 128 tile kernel; 128 / 129 /
# 257: one full row tile, one row past it, two tiles and one row
@pytest.mark.parametrize("M", [1, 7, 16, 17, 128, 129, 130, 257])
@pytest.mark.parametrize("N,K", [(48, 144), (272, 400)])
def test_w4a8_ragged(M, N, K):
    g = wl.rng(10, N, K)
    w = wl.int4_weight(g, N, K)
    pw = bql.prepack_weight(dev(wl.pack_int4(w).reshape(N, K // 2)), "int4_channel",
                            scales=dev16(wl.w4a8_channel_scales(g, N), "f16"))
    aq = g.integers(-127, 128, (M, K), dtype=np.int8)
    acc = bql.w4a8_linear(dev(aq), None, pw, out_dtype=torch.int32)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc).astype(np.int64), oracle.w4a8_acc(aq, w))


@pytest.mark.parametrize("M", [1, 3, 5, 16])
def test_small_m_split_k(M):
    """N = 256, K = 34816: the small-M kernels split K eight ways (34 k-tiles
    per split, so each wave's last weight batch lies partly past its split's
    range) and add the partial sums in a fixed order; fp8 (fused quantization
    for M <= 4), W8A16 and W4A8."""
    N, K = 256, 34816
    _fp8_case(3, 12, M, N, K, "bf16", False, "channels", torch.bfloat16)
    g = wl.rng(9, N, K, 12)
    bits = wl.weight(g, N, K, "f16")
    pw = bql.prepack_weight(dev16(bits, "f16"), "fp8_channel")
    codes, s = oracle.quant_per_row(oracle.decode_input(bits, "f16"))
    a_bits = wl.activation(wl.rng(9, M, 12), M, K, "f16")
    y = bql.w8a16_linear(dev16(a_bits, "f16"), pw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_close(host_f64(y), oracle.w8a16_linear(oracle.decode_input(a_bits, "f16"), codes, s),
                 f"W8A16 split K M={M}")
    w = wl.int4_weight(g, N, K)
    pw4 = bql.prepack_weight(dev(wl.pack_int4(w).reshape(N, K // 2)), "int4_channel",
                             scales=dev16(wl.w4a8_channel_scales(g, N), "f16"))
    aq = g.integers(-127, 128, (M, K), dtype=np.int8)
    acc = bql.w4a8_linear(dev(aq), None, pw4, out_dtype=torch.int32)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc).astype(np.int64), oracle.w4a8_acc(aq, w))


def test_w8a16_split_k_infinite_activation():
    """M = 1, N = 256, K = 34816 (K split eight ways, 4352 columns each); one
    activation column, in the third split's range, is +inf.  Each output is then +-inf by the
    sign of its weight code in that column, or NaN where that code is +-0,
    as the oracle's IEEE sums give.  A split that read the column outside
    its own range would multiply it by zero weight tiles and make every
    output NaN."""
    N, K = 256, 34816
    g = np.random.Generator(np.random.PCG64(77))
    wq = _random_codes(g, (N, K))
    col = 2 * 4352 + 300
    wq[0:3, col] = [0x00, 0x80, 0x38]
    pw = bql.prepack_weight(dev(wq), "fp8_channel", scales=torch.ones(N, device=DEV))
    a = oracle.decode_input(wl.activation(wl.rng(9, 1, 13), 1, K, "f16"), "f16").astype(np.float32)
    a[0, col] = np.inf
    y = bql.w8a16_linear(dev16(wl.to_bits(a, "f16"), "f16"), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = host_f64(y)[0]
    with np.errstate(invalid="ignore"):
        want = oracle.w8a16_linear(a, wq, np.ones(N, dtype=np.float32))[0]
    assert np.isnan(want[:2]).all() and np.isposinf(want[2]) and not np.isfinite(want).any()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(want)], want[~np.isnan(want)])


def test_w4a8_extreme_values_exact():
    # every product at its extreme: -127 * -8 * 16 per term, K = 8192
    N, K, M = 32, 8192, 17
    w = np.full((N, K), -8, dtype=np.int8)
    w[1::2] = 7
    aq = np.full((M, K), -127, dtype=np.int8)
    aq[::3] = 127
    pw = bql.prepack_weight(dev(wl.pack_int4(w).reshape(N, K // 2)), "int4_channel",
                            scales=torch.ones(N, device=DEV))
    for m in (M, 1):
        acc = bql.w4a8_linear(dev(aq[:m]), None, pw, out_dtype=torch.int32)
        torch.cuda.synchronize()
        assert np.array_equal(host(acc).astype(np.int64), oracle.w4a8_acc(aq[:m], w))


@pytest.mark.parametrize("M,K", [(2, 1024), (16, 1024), (16, 4096)])
@pytest.mark.parametrize("kind", ["nan", "inf"])
def test_small_m_nonfinite_activation(kind, M, K):
    """A NaN or an infinity in A at small M (fused quantization at M = 2 and
    M = 16, K = 1024; the amax pass and cast at M = 16, K = 4096): the
    scale is NaN or infinite as the oracle's, and the infinity's or NaN's
    code (NaN) makes every output NaN, as the oracle's IEEE sums give."""
    N = 1024
    g = wl.rng(13, M, K)
    a = oracle.decode_input(wl.activation(g, M, K, "bf16", "channels"), "bf16").astype(np.float32)
    a[M // 2, K // 3] = np.nan if kind == "nan" else np.inf
    bits = wl.to_bits(a, "bf16")
    pw = bql.prepack_weight(dev16(wl.weight(g, N, K, "bf16"), "bf16"), "fp8_tensor")
    sa = torch.empty(1, dtype=torch.float32, device=DEV)
    y = bql.fp8_linear(dev16(bits, "bf16"), pw, a_scale=sa, out_dtype=torch.float32)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):
        _, s_ref = oracle.quant_per_tensor(oracle.decode_input(bits, "bf16"))
    got = host(sa)[0]
    assert (np.isnan(got) and np.isnan(s_ref)) or got == s_ref
    assert np.isnan(host_f64(y)).all()


def test_m_zero_is_a_no_op():
    W = _weights(1, 0, 1024, 1024, "f16", False)
    pw = _packed(1, 0, 1024, 1024, "f16", False)
    y = bql.fp8_linear(torch.empty((0, 1024), dtype=torch.float16, device=DEV), pw,
                       out_dtype=torch.float16)
    assert y.shape == (0, 1024)


# ------------------------------------------- scales, pre-quantized input, determinism

def _random_codes(g, shape):
    c = g.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38
    return c


@pytest.mark.parametrize("M", [4, 200])
def test_prequantized_input_and_scale_interleave(M):
    # A and W given as E4M3 codes; per-channel scales 2^((n mod 8) - 4)
    # reveal any column that receives another column's scale.
    g = np.random.Generator(np.random.PCG64(33))
    N, K = 272, 384
    aq = _random_codes(g, (M, K))
    wq = _random_codes(g, (N, K))
    sa = np.float32(0.37)
    s_ch = np.exp2((np.arange(N) % 8) - 4).astype(np.float32)
    pw_t = bql.prepack_weight(dev(wq), "fp8_tensor", scales=torch.ones(1, device=DEV))
    pw_c = bql.prepack_weight(dev(wq), "fp8_channel", scales=dev(s_ch))
    pw_e = bql.prepack_weight(dev(wq), "fp8_channel", scales=torch.ones(N, device=DEV))
    a_t = dev(aq).view(torch.float8_e4m3fn)
    sa_t = torch.tensor([sa], device=DEV)
    y_t = bql.fp8_linear(a_t, pw_t, a_scale=sa_t, out_dtype=torch.bfloat16)
    y_c = bql.fp8_linear(a_t, pw_c, a_scale=sa_t, out_dtype=torch.bfloat16)
    y_e = bql.fp8_linear(a_t, pw_e, a_scale=sa_t, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # equal channel scales == per-tensor, bit for bit
    assert torch.equal(y_t, y_e)
    # power-of-two channel scales act exactly on their own column
    assert torch.equal(y_c.float(), y_t.float() * torch.from_numpy(s_ch).to(DEV)[None, :])
    y_ref = oracle.fp8_linear(aq, sa, wq, s_ch)
    assert_close(host_f64(y_c), y_ref, f"pre-quantized M={M}")


@pytest.mark.parametrize("M,N,K", [(300, 1040, 400), (2064, 2192, 400)])
def test_prequantized_rowmajor_and_packed_tile_paths(M, N, K):
    # E4M3 A at M > 16 in exact mode: up to 256 output tiles of 128x128 the
    # k-split kernel gathers A row-major where it is, above that A is first
    # repacked into operand tiles; ragged M and K (K = 3 * 128 + 16) on both.
    g = np.random.Generator(np.random.PCG64(M + N))
    aq = _random_codes(g, (M, K))
    wq = _random_codes(g, (N, K))
    sa = np.float32(0.011)
    sw = (g.uniform(0.5, 2.0, size=N) * 2.0 ** -6).astype(np.float32)
    pw = bql.prepack_weight(dev(wq), "fp8_channel", scales=dev(sw))
    y = bql.fp8_linear(dev(aq).view(torch.float8_e4m3fn), pw, a_scale=torch.tensor([sa], device=DEV),
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = rows_for(M, 7 + M, 40)
    assert_close(host_f64(y)[rows], oracle.fp8_linear(aq, sa, wq, sw, rows=rows),
                 f"pre-quantized tile path M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [1, 3, 16])
def test_prequantized_small_m_half_tiles(M):
    # Pre-quantized A on the small-M path is read row-major; K = 144 leaves
    # the second 16-byte half of some lanes' 32-k chunk past K (zeros).
    g = np.random.Generator(np.random.PCG64(34 + M))
    N, K = 48, 144
    aq = _random_codes(g, (M, K))
    wq = _random_codes(g, (N, K))
    sa, sw = np.float32(0.5), np.float32(0.25)
    pw = bql.prepack_weight(dev(wq), "fp8_tensor", scales=torch.tensor([sw], device=DEV))
    for fast in (False, True):
        y = bql.fp8_linear(dev(aq).view(torch.float8_e4m3fn), pw, a_scale=torch.tensor([sa], device=DEV),
                           out_dtype=torch.float32, fast_accum=fast)
        torch.cuda.synchronize()
        y_ref = oracle.fp8_linear(aq, sa, wq, np.array([sw], dtype=np.float32))
        if fast:
            abs_sum = oracle.fp8_acc(aq & 0x7F, wq & 0x7F) * np.float64(sa) * np.float64(sw)
            assert_fast_bound(host_f64(y), y_ref, abs_sum, f"pre-quantized small M={M} fast")
        else:
            assert_close(host_f64(y), y_ref, f"pre-quantized small M={M}")


@pytest.mark.parametrize("fast", [False, True])
@pytest.mark.parametrize("M", [1, 16, 1024])
def test_deterministic(M, fast):
    N, K = 4096, 4096
    pw = _packed(3, 1, N, K, "bf16", False)
    a = dev16(wl.activation(wl.rng(3, 1, M, 3), M, K, "bf16", "channels"), "bf16")
    y1 = bql.fp8_linear(a, pw, out_dtype=torch.bfloat16, fast_accum=fast)
    y2 = bql.fp8_linear(a, pw, out_dtype=torch.bfloat16, fast_accum=fast)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("M", [16, 64])
def test_every_code_decodes_exactly(M):
    # Column k=5 of W holds every finite E4M3 code once (channel n = code
    # index); every row of A is 1.0 at k=5 and 0 elsewhere, so with unit
    # scales and fp32 output Y[m, n] must be exactly dec(code n) on every
    # path: exact and fast fp8 (small-M and tiled kernels) and W8A16.
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    N, K = 256, 160
    wq = np.zeros((N, K), dtype=np.uint8)
    wq[:codes.size, 5] = codes
    want = np.zeros(N)
    want[:codes.size] = [oracle.e4m3_decode(int(c)) for c in codes]
    aq = np.zeros((M, K), dtype=np.uint8)
    aq[:, 5] = 0x38
    one = torch.ones(1, device=DEV)
    pw = bql.prepack_weight(dev(wq), "fp8_channel", scales=torch.ones(N, device=DEV))
    for fast in (False, True):
        y = bql.fp8_linear(dev(aq).view(torch.float8_e4m3fn), pw, a_scale=one,
                           out_dtype=torch.float32, fast_accum=fast)
        torch.cuda.synchronize()
        assert np.array_equal(host(y), np.broadcast_to(want, (M, N)).astype(np.float32)), fast
    a16 = np.zeros((M, K), dtype=np.float32)
    a16[:, 5] = 1.0
    y = bql.w8a16_linear(dev16(wl.to_bits(a16, "f16"), "f16"), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(host(y), np.broadcast_to(want, (M, N)).astype(np.float32))
