"""Re-derives tests/golden/rmsnorm_worked.txt with exact rational arithmetic.

The worked rows of RMSNorm ahead of the activation quantizers (QQQ issue
#15, the answer on online activation quantization fused into an
element-wise kernel such as rmsnorm) are computed here from their
definition with Python fractions: every fp64 and fp32 rounding of the
stated precision chain is done explicitly on exact rationals, the square
root is correctly rounded by comparing with squared midpoints, and the
E4M3 code is the nearest OCP E4M3 value (ties to the even code, saturation
at 448) found by scanning the 127 non-negative finite values.  Nothing here
imports the oracle, so the golden file is pinned by a derivation that
shares no code with the function it pins.  CPU only.
"""
from __future__ import annotations

import os
import struct
from fractions import Fraction as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rmsnorm_worked.txt")


def _round_binary(v: F, mant_bits: int, emin: int) -> F:
    """Nearest binary float with `mant_bits` significand bits (ties to
    even), exponent floor `emin` (gradual underflow)."""
    if v == 0:
        return F(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = F(2) ** (e - mant_bits + 1)
    q = a / ulp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def f32(v: F) -> F:
    return _round_binary(v, 24, -126)


def f64(v: F) -> F:
    return _round_binary(v, 53, -1022)


def sqrt_f64(v: F) -> F:
    """Correctly rounded fp64 square root of a positive rational."""
    # integer square root at a scale that leaves ample guard bits, then the
    # fp64 neighbours of it are decided against squared midpoints exactly
    scale = 200
    n = (v.numerator << (2 * scale)) // v.denominator
    r = F(_isqrt(n), 1 << scale)
    x = f64(r)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while F(2) ** e > x:
        e -= 1
    ulp = F(2) ** (e - 52)
    for cand in (x - ulp, x, x + ulp):
        lo, hi = cand - ulp / 2, cand + ulp / 2
        # the square of a midpoint (a 54-bit significand) is never the fp64
        # value v, so there are no ties here
        assert v != lo * lo and v != hi * hi
        if lo * lo < v < hi * hi:
            return cand
    raise AssertionError("square root bracket not found")


def _isqrt(n: int) -> int:
    x = 1 << ((n.bit_length() + 1) // 2)
    while True:
        y = (x + n // x) // 2
        if y >= x:
            return x
        x = y


def _e4m3_values():
    out = {}
    for c in range(127):
        e, m = c >> 3, c & 7
        out[c] = F(m, 8) * F(2) ** -6 if e == 0 else (1 + F(m, 8)) * F(2) ** (e - 7)
    return out


E4M3 = _e4m3_values()


def e4m3(v: F) -> int:
    sign = 0x80 if v < 0 else 0
    a = abs(v)
    if a >= 448:
        return sign | 0x7E
    lo = max(c for c in E4M3 if E4M3[c] <= a)
    mid = (E4M3[lo] + E4M3[lo + 1]) / 2
    c = lo + 1 if a > mid or (a == mid and lo % 2 == 1) else lo
    return sign | c


def rint_even(v: F) -> int:
    fl = v.numerator // v.denominator
    rem = v - fl
    return fl + (1 if rem > F(1, 2) or (rem == F(1, 2) and fl % 2) else 0)


def f32_bits(v: F) -> int:
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def derive(x, g, eps, K):
    """r, y, and both quantizers' scales and codes of one row."""
    x = [F(t) for t in x] + [F(0)] * (K - len(x))
    g = [F(t) for t in g] + [F(1)] * (K - len(g))
    ss = sum(t * t for t in x)                     # squares of 16-bit values: exact
    ms = f64(ss / K)
    d = f64(ms + F(eps))
    root = sqrt_f64(d)
    r = f32(f64(1 / root))
    y = [f32(f32(t * r) * gg) for t, gg in zip(x, g)]
    amax = max(abs(t) for t in y)
    s8 = f32(amax / 127) if amax else F(1)
    q8 = [max(-127, min(127, rint_even(f32(t / s8)))) for t in y]
    sf = f32(amax / 448) if amax else F(1)
    qf = [e4m3(f32(t / sf)) for t in y]
    return r, y, s8, q8, sf, qf


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([p.split() for p in line.split("|")])
    return rows


def test_golden_rows_rederived_exactly():
    rows = _golden()
    n = 0
    for i in range(0, len(rows), 3):
        head, xs, gs, rbits, ybits = rows[i]
        K, eps = int(head[1]), F(head[2])
        r, y, s8, q8, sf, qf = derive([F(t) for t in xs], [F(t) for t in gs], eps, K)
        assert f32_bits(r) == int(rbits[0], 16)
        assert [f32_bits(t) for t in y[:len(ybits)]] == [int(b, 16) for b in ybits]
        _, s8_g, c8_g = rows[i + 1]
        assert f32_bits(s8) == int(s8_g[0], 16)
        assert q8[:len(c8_g)] == [int(c) for c in c8_g]
        _, sf_g, cf_g = rows[i + 2]
        assert f32_bits(sf) == int(sf_g[0], 16)
        assert qf[:len(cf_g)] == [int(c, 16) for c in cf_g]
        n += 1
    assert n == 2


def test_derivation_helpers_on_known_values():
    # the helpers themselves against values fixed by IEEE arithmetic
    assert f32(F(1, 10)) == F(13421773, 2 ** 27)           # fp32(0.1)
    assert f64(F(1, 3)) == F(6004799503160661, 2 ** 54)    # fp64(1/3)
    assert sqrt_f64(F(4)) == 2 and sqrt_f64(F(25, 16)) == F(5, 4)
    assert sqrt_f64(F(2)) == F(6369051672525773, 2 ** 52)   # fp64(sqrt 2)
    assert e4m3(F(1)) == 0x38 and e4m3(F(-448)) == 0xFE and e4m3(F(500)) == 0x7E
    assert e4m3(F(17, 16)) == 0x38   # 1.0625: tie between 1.0 and 1.125 -> even
    assert e4m3(F(19, 16)) == 0x3A   # 1.1875: tie between 1.125 and 1.25 -> even
    assert rint_even(F(5, 2)) == 2 and rint_even(F(-5, 2)) == -2 and rint_even(F(7, 2)) == 4
