"""Pins of the oracle's per-group weight-only int4 linear (QQQ issue #15's
"awq-g128" and "marlin-g128" columns, read as fp16 activations, int4
weights, one scale per output channel and 128-k group, no zero point):
exact rational brute force on small shapes (a ragged last group too),
reduction to a numpy fp64 matmul when every group of a channel has the same
scale, agreement with the (separately pinned) per-group W4A8 oracle on
integer activations, and group locality.  CPU only."""
from fractions import Fraction

import numpy as np

import oracle
import workloads as wl


def _case(seed, M, N, K, group=128):
    g = np.random.Generator(np.random.PCG64(seed))
    # fp16 activations (their fp32 values), outliers included
    a = oracle.decode_input(wl.activation(g, M, K, "f16", "entries"), "f16").reshape(M, K)
    w4 = g.integers(-8, 8, size=(N, K), dtype=np.int8)
    G = -(-K // group)
    sw = (g.uniform(0.5, 2.0, size=(N, G)) * 2.0 ** -8).astype(np.float32)
    return a, w4, sw


def test_bruteforce_fractions():
    for seed, (M, N, K, group) in enumerate([(2, 3, 256, 128), (3, 2, 200, 128), (2, 2, 48, 16)]):
        a, w4, sw = _case(10 + seed, M, N, K, group)
        y = oracle.w4a16_group_linear(a, w4, sw, group=group)
        G = -(-K // group)
        for m in range(M):
            for n in range(N):
                exact = Fraction(0)
                for gi in range(G):
                    part = sum(Fraction(float(a[m, k])) * int(w4[n, k])
                               for k in range(gi * group, min((gi + 1) * group, K)))
                    exact += Fraction(float(sw[n, gi])) * part
                # the group sums are exact in fp64 (every product of an
                # fp16 value and an int4 is a multiple of 2^-24 below 2^29);
                # only the scale products and the sum over a few groups round
                assert abs(Fraction(y[m, n]) - exact) <= (abs(exact) + 1) * Fraction(1, 2 ** 48)


def test_equal_group_scales_reduce_to_matmul():
    a, w4, _ = _case(1, 5, 12, 512)
    s = np.random.Generator(np.random.PCG64(2)).uniform(0.5, 2.0, 12).astype(np.float32)
    y = oracle.w4a16_group_linear(a, w4, np.repeat(s[:, None], 4, axis=1))
    ref = (a.astype(np.float64) @ w4.astype(np.float64).T) * s.astype(np.float64)[None, :]
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_matches_w4a8_group_on_integer_activations():
    # integer activations in [-127, 127] are exact fp16 values: with unit
    # activation scales the per-group W4A8 oracle computes the same sums
    g = np.random.Generator(np.random.PCG64(3))
    aq = g.integers(-127, 128, size=(4, 384), dtype=np.int8)
    w4 = g.integers(-8, 8, size=(6, 384), dtype=np.int8)
    sw = (g.uniform(0.5, 2.0, size=(6, 3)) * 2.0 ** -8).astype(np.float32)
    y16 = oracle.w4a16_group_linear(aq.astype(np.float32), w4, sw)
    y8 = oracle.w4a8_group_linear(aq, np.ones(4, np.float32), w4, sw)
    assert np.array_equal(y16, y8)


def test_group_locality_and_scale_placement():
    a, w4, sw = _case(4, 3, 8, 512)
    w4 = w4.copy()
    w4[:, :256] = 0
    w4[:, 384:] = 0          # only group 2 carries weights
    y = oracle.w4a16_group_linear(a, w4, sw)
    sw2 = sw.copy()
    sw2[:, [0, 1, 3]] *= 3.7  # other groups' scales do not matter
    assert np.array_equal(oracle.w4a16_group_linear(a, w4, sw2), y)
    sw3 = sw.copy()
    sw3[:, 2] *= 2            # that group's scale scales Y exactly
    assert np.array_equal(oracle.w4a16_group_linear(a, w4, sw3), 2 * y)
    sw4 = sw.copy()
    sw4[3, 2] *= 4            # a channel's scale acts on its own column only
    y4 = oracle.w4a16_group_linear(a, w4, sw4)
    assert np.array_equal(y4[:, 3], 4 * y[:, 3])
    assert np.array_equal(np.delete(y4, 3, axis=1), np.delete(y, 3, axis=1))
