"""Pins of the CPU oracle to facts outside itself (runs without a GPU).

Each test checks the oracle against something it does not compute itself:
hand-derived values of the OCP E4M3 format, library routines (torch's CPU
float8_e4m3fn conversion, numpy float16 / int64 matmul), exact rational
brute force, closed forms and invariants.  Chosen so that a dropped term, a
wrong sign or index, or a transposed operand in the oracle fails one.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line.split()


# --------------------------------------------------------------- E4M3

def test_decode_golden_values():
    n = 0
    for tok in _golden_lines("e4m3_values.txt"):
        if tok[0] != "decode":
            continue
        code, val = int(tok[1], 16), float(tok[2])
        got = oracle.e4m3_decode(code)
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)
        n += 1
    assert n >= 10


def test_encode_golden_values():
    n = 0
    for tok in _golden_lines("e4m3_values.txt"):
        if tok[0] != "encode":
            continue
        assert oracle.e4m3_encode(float(tok[1])) == int(tok[2], 16), tok
        n += 1
    assert n >= 15


def test_decode_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = oracle.e4m3_decode_table()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.all(np.isnan(got[nan]))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_fnuz_catchers():
    # The MI300-era FNUZ variant has max 240 (bias 8) and NaN at 0x80.
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x80) == 0.0 and math.copysign(1, oracle.e4m3_decode(0x80)) < 0


def test_roundtrip_all_finite_codes():
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c, hex(c)


def _torch_cast(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_cast_below_overflow():
    # torch's CPU cast rounds to nearest even but does not saturate: it
    # agrees with the saturating definition wherever |v| <= 464.
    g = np.random.Generator(np.random.PCG64(7))
    mags = np.exp2(g.uniform(-14, 9, 20000)).astype(np.float32)
    v = mags * np.where(g.random(20000) < 0.5, -1, 1).astype(np.float32)
    # every finite code value, every midpoint between neighbours, and one
    # fp32 ulp either side of each midpoint
    tab = oracle.e4m3_decode_table()[:0x7F]
    mids = ((tab[:-1] + tab[1:]) / 2).astype(np.float32)
    extra = np.concatenate([tab.astype(np.float32), mids,
                            np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    v = np.concatenate([v, extra, -extra]).astype(np.float32)
    v = v[np.abs(v) <= 464]
    got = oracle.e4m3_encode_array(v.astype(np.float64))
    assert np.array_equal(got, _torch_cast(v))


def test_encode_saturates_and_keeps_sign():
    for v in [448.0, 449.0, 463.9, 464.0, 480.0, 1e4, 3.4e38, math.inf]:
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE
    assert oracle.e4m3_encode(-1e-30) == 0x80
    assert oracle.e4m3_encode(1e-30) == 0x00


# ------------------------------------------------------------ 16-bit inputs

def test_f16_decode_all_patterns_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = oracle.decode_input(bits, "f16")
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.all(np.isnan(got[~fin]))


def test_bf16_decode_all_patterns_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.decode_input(bits, "bf16")
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))


def test_bf16_rounding_of_generator_vs_torch():
    # the input generator's fp32 -> bf16 rounding matches torch's
    g = np.random.Generator(np.random.PCG64(3))
    x = (g.standard_normal(10000) * np.exp2(g.uniform(-20, 20, 10000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.f32_to_bf16_bits(x), ref)


# ---------------------------------------------------------- quantizers

def test_quant_worked_examples():
    n = 0
    for tok in _golden_lines("quant_worked.txt"):
        line = " ".join(tok[1:])
        parts = [p.split() for p in line.split("|")]
        ins, scale, outs = parts[-3:]
        if tok[0] == "quant":
            dtype, vals = ins[0], np.array([float(t) for t in ins[1:]], dtype=np.float32)
            x = oracle.decode_input(wl.to_bits(vals, dtype), dtype) if dtype != "f32" else vals
            q, s = oracle.quant_per_tensor(x)
            assert s == np.float32(float(scale[0]))
            assert list(q) == [int(c, 16) for c in outs]
        elif tok[0] in ("perrow", "withscales"):
            dtype, cols = tok[1], int(tok[2])
            vals = np.array([float(t) for t in ins], dtype=np.float32)
            x = oracle.decode_input(wl.to_bits(vals, dtype), dtype) if dtype != "f32" else vals
            x = x.reshape(-1, cols)
            sc = np.array([float(t) for t in scale], dtype=np.float32)
            if tok[0] == "perrow":
                q, s = oracle.quant_per_row(x)
                assert np.array_equal(s, sc)
            else:
                q = oracle.quant_with_scales(x, sc)
            assert list(q.ravel()) == [int(c, 16) for c in outs]
        else:
            x = np.array([[float(t) for t in ins]], dtype=np.float32)
            q, s = oracle.int8_quant_per_token(x)
            assert s[0] == np.float32(float(scale[0]))
            assert list(q[0]) == [int(c) for c in outs]
        n += 1
    assert n == 8


def _sample(seed, M=8, K=256):
    g = np.random.Generator(np.random.PCG64(seed))
    return (g.standard_normal((M, K)) * np.where(g.random((M, K)) < 0.02, 20, 1)).astype(np.float32)


def test_quant_amax_element_maps_to_max_code():
    x = _sample(1)
    q, s = oracle.quant_per_tensor(x)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q[i] == (0xFE if x[i] < 0 else 0x7E)
    assert s == np.float32(np.abs(x).max() / np.float32(448))


def test_quant_power_of_two_scaling_invariance():
    x = _sample(2)
    q0, s0 = oracle.quant_per_tensor(x)
    for j in (-5, -1, 1, 7):
        q, s = oracle.quant_per_tensor((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(q, q0)
        assert s == np.float32(s0 * np.float32(2.0 ** j))


def test_quant_negation_flips_sign_bit_only():
    x = _sample(3)
    q0, s0 = oracle.quant_per_tensor(x)
    q1, s1 = oracle.quant_per_tensor(-x)
    assert s0 == s1
    assert np.array_equal(q1, q0 ^ 0x80)


def test_quant_codes_are_nearest_to_scaled_input():
    # brute force: the chosen code is a nearest E4M3 value to fp32(x/s)
    x = _sample(4, 4, 64)
    q, s = oracle.quant_per_tensor(x)
    tab = oracle.e4m3_decode_table()
    fin = np.array([c for c in range(256) if c & 0x7F != 0x7F])
    for xi, qi in zip(x.ravel(), q.ravel()):
        r = float(np.float32(xi) / np.float32(s))
        best = np.min(np.abs(tab[fin] - r))
        assert abs(tab[qi] - r) == best


def test_quant_nonfinite_amax_follows_torch():
    # the amax of a tensor holding a NaN is NaN and of one holding an
    # infinity is infinite, as torch computes it; the scale amax / 448 is
    # then NaN (every code the NaN code) or infinite (every finite x / s a
    # zero of x's sign, inf / inf the NaN code)
    x = _sample(6)
    y = x.copy()
    y[1, 7] = np.nan
    assert torch.isnan(torch.from_numpy(y).abs().max())
    q, s = oracle.quant_per_tensor(y)
    assert np.isnan(s) and np.all((q & 0x7F) == 0x7F)
    y = x.copy()
    y[2, 3] = -np.inf
    assert torch.isinf(torch.from_numpy(y).abs().max())
    q, s = oracle.quant_per_tensor(y)
    assert np.isposinf(s)
    fin = np.isfinite(y)
    assert np.array_equal(q[fin], np.where(np.signbit(y[fin]), 0x80, 0x00))
    assert (q[2, 3] & 0x7F) == 0x7F
    # per row: only the row holding the NaN is NaN; the others are
    # quantized as they are alone
    y = x.copy()
    y[3, 0] = np.nan
    q, s = oracle.quant_per_row(y)
    for n in range(y.shape[0]):
        if n == 3:
            assert np.isnan(s[n]) and np.all((q[n] & 0x7F) == 0x7F)
        else:
            qn, sn = oracle.quant_per_tensor(y[n])
            assert np.array_equal(q[n], qn) and s[n] == sn, n


def test_per_row_with_equal_rows_equals_per_tensor():
    x = _sample(5)
    amax = np.abs(x).max()
    x[:, 0] = amax  # every row has the same amax
    qt, st = oracle.quant_per_tensor(x)
    qr, sr = oracle.quant_per_row(x)
    assert np.all(sr == st)
    assert np.array_equal(qt, qr)
    assert np.array_equal(oracle.quant_with_scales(x, np.array([st])), qt)


def _rows_scaled_by_row_index(seed, rows=16, cols=96):
    """Rows n = base * 2^(n mod 8) (exact in fp32): every row has the same
    codes and row n's scale is exactly 2^(n mod 8) times row 0's."""
    g = np.random.Generator(np.random.PCG64(seed))
    base = (g.standard_normal(cols) * np.where(g.random(cols) < 0.05, 20, 1)).astype(np.float32)
    mult = np.exp2(np.arange(rows) % 8).astype(np.float32)
    return (base[None, :] * mult[:, None]).astype(np.float32), mult


def test_per_row_quant_uses_each_rows_own_amax():
    # a global amax, or the amax of another row, gives other codes for all
    # but one of these rows
    x, mult = _rows_scaled_by_row_index(21)
    q, s = oracle.quant_per_row(x)
    for n in range(x.shape[0]):
        assert np.array_equal(q[n], q[0]), n
        assert s[n] == np.float32(s[0] * mult[n]), n
    # and each row is quantized exactly as the (hand-pinned) per-tensor
    # quantizer quantizes that row alone
    g = np.random.Generator(np.random.PCG64(22))
    y = (g.standard_normal((12, 80)) * np.exp2(g.integers(-6, 7, (12, 1)))).astype(np.float32)
    y[5] = 0.0  # an all-zero row takes scale 1
    q, s = oracle.quant_per_row(y)
    for n in range(y.shape[0]):
        qn, sn = oracle.quant_per_tensor(y[n])
        assert np.array_equal(q[n], qn) and s[n] == sn, n
    assert s[5] == np.float32(1.0) and not q[5].any()


def test_quant_with_scales_applies_each_rows_scale():
    # position-revealing scales: row n divided by its own 2^(n mod 8) * s0
    # gives row 0's codes on every row; any other row's scale does not
    x, mult = _rows_scaled_by_row_index(23)
    q0, s0 = oracle.quant_per_tensor(x[0])
    sc = (s0 * mult).astype(np.float32)
    q = oracle.quant_with_scales(x, sc)
    for n in range(x.shape[0]):
        assert np.array_equal(q[n], q0), n
    # the scales the per-row quantizer chose, given back, give its codes
    g = np.random.Generator(np.random.PCG64(24))
    y = (g.standard_normal((9, 64)) * np.exp2(g.integers(-4, 5, (9, 1)))).astype(np.float32)
    qr, sr = oracle.quant_per_row(y)
    assert np.array_equal(oracle.quant_with_scales(y, sr), qr)
    # and one scale for the whole matrix is the per-tensor quantizer
    qt, st = oracle.quant_per_tensor(y)
    assert np.array_equal(oracle.quant_with_scales(y, np.array([st], np.float32)), qt)


def test_int8_per_token_invariants():
    x = _sample(6)
    q, s = oracle.int8_quant_per_token(x)
    for m in range(x.shape[0]):
        i = np.argmax(np.abs(x[m]))
        assert abs(int(q[m, i])) == 127 and np.sign(q[m, i]) == np.sign(x[m, i])
        assert s[m] == np.float32(np.abs(x[m]).max() / np.float32(127))
    q2, s2 = oracle.int8_quant_per_token((x * np.float32(8)).astype(np.float32))
    assert np.array_equal(q2, q) and np.all(s2 == s * np.float32(8))
    q3, _ = oracle.int8_quant_per_token(-x)
    assert np.array_equal(q3, -q)


# ------------------------------------------------------------ linears

def _frac_decode(c):
    v = oracle.e4m3_decode(c)
    return Fraction(v)


def test_fp8_linear_bruteforce_fractions():
    g = np.random.Generator(np.random.PCG64(11))
    for (M, N, K) in [(1, 1, 1), (2, 3, 5), (3, 8, 8), (8, 2, 7)]:
        aq = g.integers(0, 256, (M, K), dtype=np.uint8)
        wq = g.integers(0, 256, (N, K), dtype=np.uint8)
        aq[(aq & 0x7F) == 0x7F] = 0x38
        wq[(wq & 0x7F) == 0x7F] = 0x38
        sa = np.float32(g.uniform(0.1, 3))
        sw = g.uniform(0.1, 3, N).astype(np.float32)
        y = oracle.fp8_linear(aq, sa, wq, sw)
        for m in range(M):
            for n in range(N):
                acc = sum(_frac_decode(int(aq[m, k])) * _frac_decode(int(wq[n, k])) for k in range(K))
                ref = Fraction(float(sa)) * Fraction(float(sw[n])) * acc
                assert abs(Fraction(y[m, n]) - ref) <= abs(ref) * Fraction(1, 2 ** 50)
        acc = oracle.fp8_acc(aq, wq)
        for m in range(M):
            for n in range(N):
                exact = sum(_frac_decode(int(aq[m, k])) * _frac_decode(int(wq[n, k])) for k in range(K))
                assert Fraction(acc[m, n]) == exact


def test_fp8_linear_integer_matmul_reduction():
    # Integers |v| <= 16 are exact in E4M3, so with unit scales the linear is
    # an integer matmul (numpy int64), transposed operand convention Y = A W^T.
    g = np.random.Generator(np.random.PCG64(12))
    M, N, K = 5, 7, 64
    ai = g.integers(-16, 17, (M, K))
    wi = g.integers(-16, 17, (N, K))
    aq = oracle.e4m3_encode_array(ai.astype(np.float64))
    wq = oracle.e4m3_encode_array(wi.astype(np.float64))
    y = oracle.fp8_linear(aq, 1.0, wq, np.float32(1.0))
    assert np.array_equal(y, (ai @ wi.T).astype(np.float64))
    # and a non-square check of row/column placement
    y2 = oracle.fp8_linear(aq[:2], 1.0, wq[:3], np.float32(1.0))
    assert np.array_equal(y2, (ai[:2] @ wi[:3].T).astype(np.float64))


def test_fp8_linear_scales_land_on_their_column():
    # position-revealing per-channel scales: column n is scaled by sW[n]
    g = np.random.Generator(np.random.PCG64(13))
    M, N, K = 3, 16, 32
    aq = oracle.e4m3_encode_array(g.integers(-8, 9, (M, K)).astype(np.float64))
    wq = oracle.e4m3_encode_array(g.integers(-8, 9, (N, K)).astype(np.float64))
    sw = np.exp2((np.arange(N) % 8) - 4).astype(np.float32)
    y1 = oracle.fp8_linear(aq, 1.0, wq, np.float32(1.0))
    y = oracle.fp8_linear(aq, 0.5, wq, sw)
    assert np.array_equal(y, 0.5 * y1 * sw.astype(np.float64)[None, :])


def test_fp8_linear_k_permutation_invariance_and_rows():
    g = np.random.Generator(np.random.PCG64(14))
    M, N, K = 6, 5, 96
    aq = g.integers(0, 0x7E, (M, K), dtype=np.uint8) | (g.integers(0, 2, (M, K), dtype=np.uint8) << 7)
    wq = g.integers(0, 0x7E, (N, K), dtype=np.uint8) | (g.integers(0, 2, (N, K), dtype=np.uint8) << 7)
    perm = g.permutation(K)
    y = oracle.fp8_linear(aq, 0.25, wq, np.float32(2.0))
    assert np.array_equal(y, oracle.fp8_linear(aq[:, perm], 0.25, wq[:, perm], np.float32(2.0)))
    rows = np.array([4, 1], dtype=np.int64)
    assert np.array_equal(oracle.fp8_linear(aq, 0.25, wq, np.float32(2.0), rows=rows), y[rows])


def test_per_channel_equal_scales_equals_per_tensor():
    g = np.random.Generator(np.random.PCG64(15))
    aq = g.integers(0, 0x7E, (4, 48), dtype=np.uint8)
    wq = g.integers(0, 0x7E, (9, 48), dtype=np.uint8)
    s = np.float32(0.0123)
    yt = oracle.fp8_linear(aq, 0.5, wq, s)
    yc = oracle.fp8_linear(aq, 0.5, wq, np.full(9, s, dtype=np.float32))
    assert np.array_equal(yt, yc)


def test_fp8_output_codes_vs_torch_cast():
    g = np.random.Generator(np.random.PCG64(16))
    y = g.standard_normal(5000) * 3
    c = oracle.fp8_output(y, 0.01)
    v = (y / 0.01)
    ok = np.abs(v) <= 400
    # where y/os is exactly an fp32, torch's RNE cast is an independent route
    v32 = v.astype(np.float32)
    exact = ok & (v32.astype(np.float64) == v)
    assert np.array_equal(c[exact], _torch_cast(v32[exact]))
    assert np.all(c[np.abs(v) > 448] & 0x7F == 0x7E)


def test_w8a16_vs_float64_matmul():
    g = np.random.Generator(np.random.PCG64(17))
    M, N, K = 3, 10, 128
    a = g.standard_normal((M, K)).astype(np.float16).astype(np.float32)
    wq = g.integers(0, 0x7E, (N, K), dtype=np.uint8) | (g.integers(0, 2, (N, K), dtype=np.uint8) << 7)
    sw = g.uniform(0.5, 2, N).astype(np.float32)
    wdec = torch.from_numpy(wq).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = (a.astype(np.float64) @ wdec.T) * sw.astype(np.float64)[None, :]
    y = oracle.w8a16_linear(a, wq, sw)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_int4_packing_and_w4a8_acc_vs_int_matmul():
    g = np.random.Generator(np.random.PCG64(18))
    M, N, K = 4, 12, 64
    w = wl.int4_weight(g, N, K)
    packed = wl.pack_int4(w)
    # the logical packing: low nibble is the even k
    assert (packed[0] & 15) == (w[0, 0] & 15) and (packed[0] >> 4) == (w[0, 1] & 15)
    assert np.array_equal(oracle.unpack_int4(packed, N, K), w)
    aq = g.integers(-127, 128, (M, K), dtype=np.int8)
    acc = oracle.w4a8_acc(aq, w)
    assert np.array_equal(acc, aq.astype(np.int64) @ w.astype(np.int64).T)
    # widening int4 -> int8 by *16 then dividing the int32 sum by 16 is exact
    assert np.array_equal((aq.astype(np.int64) @ (16 * w.astype(np.int64)).T) >> 4, acc)
    sa = g.uniform(0.01, 0.1, M).astype(np.float32)
    sw = g.uniform(0.5, 2, N).astype(np.float32)
    y = oracle.w4a8_linear(acc, sa, sw)
    assert np.allclose(y, acc * sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :], rtol=1e-15)


def test_w4a8_acc_overflow_is_refused():
    aq = np.full((1, 2 ** 22), -127, dtype=np.int8)
    w = np.full((1, 2 ** 22), -8, dtype=np.int8)
    with pytest.raises(OverflowError):
        oracle.w4a8_acc(aq, w)


def test_tolerance_rule():
    ref = np.array([1.0, -2.0, 0.0, 100.0])
    ok, worst = oracle.within_tolerance(ref * (1 + 4e-3), ref)
    assert ok and worst < 1
    ok, _ = oracle.within_tolerance(ref * (1 + 6e-3), ref)
    assert not ok
    # near-zero outputs get the floor 1e-2 * max|ref|
    ok, _ = oracle.within_tolerance(np.array([1.0, -2.0, 4e-3, 100.0]), ref)
    assert ok
