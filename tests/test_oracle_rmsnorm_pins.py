"""Pins of the oracle's RMSNorm step, the element-wise op the activation
quantizers are fused into (QQQ issue #15, the answer on online activation
quantization), against values derived by hand, torch's own rms_norm in
fp64, closed forms and invariants.  CPU only."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "rmsnorm_worked.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([p.split() for p in line.split("|")])
    return rows


def _bits(v):
    return int(np.float32(v).view(np.uint32))


def test_rmsnorm_worked_examples():
    rows = _golden_rows()
    n = 0
    i = 0
    while i < len(rows):
        head, xs, gs, rbits, ybits = rows[i]
        K, eps = int(head[1]), float(head[2])
        nx = len(xs)
        x = np.zeros((1, K), dtype=np.float32)
        x[0, :nx] = [float(t) for t in xs]
        g = np.ones(K, dtype=np.float32)
        g[:len(gs)] = [float(t) for t in gs]
        y, r = oracle.rmsnorm(x, g, eps)
        assert _bits(r[0]) == int(rbits[0], 16)
        assert [_bits(v) for v in y[0, :len(ybits)]] == [int(b, 16) for b in ybits]
        _, s8, c8 = rows[i + 1]
        q, s, _ = oracle.rmsnorm_int8_per_token(x, g, eps)
        assert _bits(s[0]) == int(s8[0], 16)
        assert list(q[0, :len(c8)]) == [int(c) for c in c8]
        _, sf, cf = rows[i + 2]
        q, s, _ = oracle.rmsnorm_fp8_per_tensor(x, g, eps)
        assert _bits(s) == int(sf[0], 16)
        assert list(q[0, :len(cf)]) == [int(c, 16) for c in cf]
        i += 3
        n += 1
    assert n == 2


def _inputs(seed, M, K, dtype):
    g = wl.rng(99, seed)
    x = oracle.decode_input(wl.activation(g, M, K, dtype, "channels"), dtype)
    w = oracle.decode_input(wl.norm_weight(g, K, dtype), dtype)
    return x, w


def test_rmsnorm_vs_torch_rms_norm():
    for seed, (M, K, dtype, eps) in enumerate([(8, 4096, "bf16", 1e-5), (5, 1024, "f16", 1e-6),
                                                (3, 48, "f16", 1e-5), (4, 8192, "bf16", 1e-2)]):
        x, w = _inputs(seed, M, K, dtype)
        y, r = oracle.rmsnorm(x, w, eps)
        x64 = torch.from_numpy(x.astype(np.float64))
        yt = torch.nn.functional.rms_norm(x64, (K,), torch.from_numpy(w.astype(np.float64)),
                                          eps=np.float32(eps).item()).numpy()
        rt = torch.rsqrt(x64.pow(2).mean(-1) + np.float32(eps).item()).numpy()
        # r: one rounding to fp32 of an fp64 chain
        assert np.all(np.abs(r - rt) <= 2.0 ** -24 * np.abs(rt) * 1.0001)
        # y: r, x*r and *g each rounded once to fp32
        assert np.all(np.abs(y - yt) <= 3.0001 * 2.0 ** -24 * np.abs(yt))


def test_rmsnorm_power_of_two_rows_are_exact():
    K = 256
    gen = np.random.Generator(np.random.PCG64(5))
    g = (gen.uniform(0.5, 1.5, K)).astype(np.float16).astype(np.float32)
    j = np.array([-9, -1, 0, 3, 11])
    x = (np.where(gen.random((j.size, K)) < 0.5, -1.0, 1.0) * 2.0 ** j[:, None]).astype(np.float32)
    y, r = oracle.rmsnorm(x, g, 0.0)
    assert np.array_equal(r, (2.0 ** -j).astype(np.float32))
    assert np.array_equal(y, np.sign(x) * g[None, :])


def test_rmsnorm_invariances():
    x, w = _inputs(7, 6, 1024, "bf16")
    y, r = oracle.rmsnorm(x, w, 0.0)
    # x * 2^j: same y, r / 2^j (exact with eps = 0)
    for j in (-7, 5):
        y2, r2 = oracle.rmsnorm(x * np.float32(2.0 ** j), w, 0.0)
        assert np.array_equal(y2, y)
        assert np.array_equal(r2 * np.float32(2.0 ** j), r)
    # negation flips y
    y3, _ = oracle.rmsnorm(-x, w, 0.0)
    assert np.array_equal(y3, -y)
    # g * 2^i scales y exactly, column by column
    scale = np.float32(2.0) ** np.arange(-3, 4, dtype=np.float32)[np.arange(1024) % 7]
    y4, _ = oracle.rmsnorm(x, w * scale, 1e-5)
    y5, _ = oracle.rmsnorm(x, w, 1e-5)
    assert np.array_equal(y4, y5 * scale)
    # permuting k permutes y (with g permuted alike); r unchanged up to the
    # summation order (admissible set)
    p = np.random.Generator(np.random.PCG64(1)).permutation(1024)
    y6, r6 = oracle.rmsnorm(x[:, p], w[p], 1e-5)
    lo, hi = oracle.rms_inv_candidates(x, 1e-5)
    assert np.all((r6 == lo) | (r6 == hi))
    same = r6 == oracle.rmsnorm(x, w, 1e-5)[1]
    assert np.array_equal(y6[same], y5[same][:, p])


def test_rms_inv_candidates_cover_other_summation_orders():
    x, _ = _inputs(11, 64, 4096, "bf16")
    eps = 1e-5
    lo, hi = oracle.rms_inv_candidates(x, eps)
    _, r = oracle.rmsnorm(x, np.ones(4096, np.float32), eps)
    assert np.all((r == lo) | (r == hi))
    x64 = x.astype(np.float64) ** 2
    for ss in (x64.sum(axis=1),                      # numpy pairwise order
               x64[:, ::-1].cumsum(axis=1)[:, -1],    # reversed sequential order
               x64.reshape(64, 64, 64).sum(axis=2).sum(axis=1)):  # blocked tree
        rr = np.array([oracle.rms_inv(s, 4096, eps) for s in ss], dtype=np.float32)
        assert np.all((rr == lo) | (rr == hi))


def test_zero_row_with_eps():
    x = np.zeros((2, 32), dtype=np.float32)
    x[1, 3] = 2.0
    g = np.ones(32, dtype=np.float32)
    q, s, r = oracle.rmsnorm_int8_per_token(x, g, 0.25)
    assert r[0] == np.float32(2.0)          # 1 / sqrt(0 + 1/4)
    assert s[0] == np.float32(1.0) and not q[0].any()
    q, s, r = oracle.rmsnorm_fp8_per_tensor(x, g, 0.25)
    assert q[1, 3] == 0x7E and np.count_nonzero(q) == 1


def test_fused_quantizers_compose_the_pinned_quantizers():
    x, w = _inputs(3, 16, 1024, "f16")
    y, r = oracle.rmsnorm(x, w, 1e-5)
    q, s, r2 = oracle.rmsnorm_int8_per_token(x, w, 1e-5)
    q0, s0 = oracle.int8_quant_per_token(y)
    assert np.array_equal(q, q0) and np.array_equal(s, s0) and np.array_equal(r, r2)
    q, s, _ = oracle.rmsnorm_fp8_per_tensor(x, w, 1e-5, r=r)
    q0, s0 = oracle.quant_per_tensor(y)
    assert np.array_equal(q, q0) and s == s0
