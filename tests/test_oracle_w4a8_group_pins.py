"""Pins of the oracle's per-group W4A8 (QQQ issue #15's "qqq-g128" columns,
read as one scale per output channel and 128-k group): reduction to the
pinned per-channel W4A8 when every group of a channel has the same scale,
exact rational brute force on small shapes (also a ragged last group), and
group locality.  CPU only."""
from fractions import Fraction

import numpy as np

import oracle


def _case(seed, M, N, K, group=128):
    g = np.random.Generator(np.random.PCG64(seed))
    aq = g.integers(-127, 128, size=(M, K), dtype=np.int8)
    w4 = g.integers(-8, 8, size=(N, K), dtype=np.int8)
    sa = g.uniform(0.001, 0.1, size=M).astype(np.float32)
    G = -(-K // group)
    sw = (g.uniform(0.5, 2.0, size=(N, G)) * 2.0 ** -8).astype(np.float32)
    return aq, w4, sa, sw


def test_equal_group_scales_reduce_to_per_channel():
    aq, w4, sa, _ = _case(1, 6, 10, 512)
    acc = oracle.w4a8_acc(aq, w4)
    # power-of-two channel scales: every step exact, so bit for bit
    s = (2.0 ** np.arange(-9, 1)).astype(np.float32)
    y_ch = oracle.w4a8_linear(acc, sa, s)
    y_g = oracle.w4a8_group_linear(aq, sa, w4, np.repeat(s[:, None], 4, axis=1))
    assert np.array_equal(y_g, y_ch)
    # general channel scales: equal up to fp64 rounding
    s = np.random.Generator(np.random.PCG64(2)).uniform(0.5, 2.0, 10).astype(np.float32)
    y_ch = oracle.w4a8_linear(acc, sa, s)
    y_g = oracle.w4a8_group_linear(aq, sa, w4, np.repeat(s[:, None], 4, axis=1))
    assert np.allclose(y_g, y_ch, rtol=1e-13, atol=0)


def test_bruteforce_fractions():
    for seed, (M, N, K, group) in enumerate([(2, 3, 256, 128), (3, 2, 192, 128), (2, 2, 48, 16)]):
        aq, w4, sa, sw = _case(10 + seed, M, N, K, group)
        y = oracle.w4a8_group_linear(aq, sa, w4, sw, group=group)
        G = -(-K // group)
        for m in range(M):
            for n in range(N):
                tot = Fraction(0)
                for gi in range(G):
                    acc = sum(int(aq[m, k]) * int(w4[n, k])
                              for k in range(gi * group, min((gi + 1) * group, K)))
                    tot += Fraction(float(sw[n, gi])) * acc
                exact = Fraction(float(sa[m])) * tot
                assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_group_locality():
    aq, w4, sa, sw = _case(3, 4, 8, 512)
    w4 = w4.copy()
    w4[:, :256] = 0          # only groups 2 and 3 carry weights
    w4[:, 384:] = 0          # only group 2
    y = oracle.w4a8_group_linear(aq, sa, w4, sw)
    sw2 = sw.copy()
    sw2[:, [0, 1, 3]] *= 3.7  # other groups' scales do not matter
    assert np.array_equal(oracle.w4a8_group_linear(aq, sa, w4, sw2), y)
    sw3 = sw.copy()
    sw3[:, 2] *= 2            # that group's scale scales Y exactly
    assert np.array_equal(oracle.w4a8_group_linear(aq, sa, w4, sw3), 2 * y)
