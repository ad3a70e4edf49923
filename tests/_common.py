"""Helpers shared by the GPU parity tests: moving seeded host arrays to the
device, sampling output rows, and the comparison rules.

The comparison rules:
  * integer/byte results (E4M3 codes, scales as bit patterns, int8 codes,
    int32 accumulators) must be identical;
  * float outputs must satisfy |got - ref| <= 5e-3 (|ref| + 1e-2 max|ref|)
    against the oracle's fp64 result;
  * an fp8 output code c is accepted when c = E4M3(v) for some v within
    that tolerance of the oracle's Y / output_scale (fp32 accumulation
    order decides codes near rounding boundaries).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads as wl

DEV = "cuda:0"
TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def dev16(bits: np.ndarray, dtype: str) -> torch.Tensor:
    """uint16 bit patterns -> fp16/bf16 device tensor of the same shape."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(DEV).view(TORCH_DT[dtype])


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rows_for(M: int, seed: int, count: int = 32) -> np.ndarray:
    """All rows when few, else first, last and a seeded sample."""
    if M <= count:
        return np.arange(M, dtype=np.int64)
    g = np.random.Generator(np.random.PCG64(seed))
    r = set(g.choice(M, size=count - 2, replace=False).tolist()) | {0, M - 1}
    return np.array(sorted(r), dtype=np.int64)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str):
    ok, worst = oracle.within_tolerance(got, ref)
    assert ok, f"{what}: worst |d|/bound = {worst:.3g}"
    say(f"  {what}: worst |d|/bound = {worst:.3g}")


def assert_fast_bound(got: np.ndarray, ref: np.ndarray, abs_sum: np.ndarray, what: str):
    """Bound for the fp8 matrix cores' own accumulation (fast mode).

    Measured on gfx950: each run of 8 consecutive-k products is added in a
    fixed-point window of 14 bit positions aligned to the exponent e of the
    largest of the 8, so each of the other 7 loses less than 2^(e-13) <=
    2^-13 * (largest) and a run errs by < 7 * 2^-13 * sum|p| < 2^-10 sum|p|.
    abs_sum is sA sW[n] sum_k |dec(a) dec(w)| per output; on top comes the
    output rounding, covered by the float tolerance."""
    tol = 5e-3 * (np.abs(ref) + 1e-2 * np.abs(ref).max()) + 2.0 ** -10 * abs_sum
    d = np.abs(got - ref)
    worst = float((d / tol).max()) if d.size else 0.0
    assert np.all(d <= tol), f"{what}: worst |d|/bound = {worst:.3g}"
    say(f"  {what}: worst |d|/fast-bound = {worst:.3g}")


def assert_fp8_out(codes: np.ndarray, v_ref: np.ndarray, what: str) -> float:
    """Acceptance of fp8 output codes; returns the exact-match fraction."""
    tab = oracle.e4m3_decode_table()
    codes = codes.astype(np.int64)
    assert not np.any((codes & 0x7F) == 0x7F), f"{what}: NaN code"
    got = tab[codes]
    tol = 5e-3 * (np.abs(v_ref) + 1e-2 * np.abs(v_ref).max())
    lo = oracle.e4m3_encode_array(v_ref - tol)
    hi = oracle.e4m3_encode_array(v_ref + tol)
    lo_v, hi_v = tab[lo.astype(np.int64)], tab[hi.astype(np.int64)]
    ok = (got >= lo_v) & (got <= hi_v)
    assert ok.all(), f"{what}: {int((~ok).sum())} fp8 codes outside the tolerance window"
    exact = float(np.mean(codes == oracle.e4m3_encode_array(v_ref).astype(np.int64)))
    say(f"  {what}: fp8 codes exact match {exact:.4f}")
    return exact


class Weights:
    """A seeded fp16/bf16 weight [N,K] with the oracle's quantization."""

    def __init__(self, cfg: int, idx: int, N: int, K: int, dtype: str, per_channel: bool):
        g = wl.rng(cfg, idx, 1)
        self.N, self.K, self.dtype = N, K, dtype
        self.bits = wl.weight(g, N, K, dtype)
        wf = oracle.decode_input(self.bits, dtype)
        if per_channel:
            self.codes, self.scales = oracle.quant_per_row(wf)
        else:
            self.codes, s = oracle.quant_per_tensor(wf)
            self.scales = np.array([s], dtype=np.float32)
        del wf


def exact_plan(M: int, N: int, K: int) -> tuple:
    """(fn, splits) of the exact fp8 tile kernel for an M x N x K linear:
    blocks of 256 rows x 32 fn columns (each wave 128 rows x fn 16-column
    strips), K split `splits` ways; (0, 1) where the 128-row kernels run
    (M <= 128).  The library's cost model in microseconds: rounds of 256
    blocks (one per CU), a tail round a little faster, a k-tile costing
    0.76 + 0.25 fn, 1.3 per block, and for K splits the fp32 partials at
    6 MB/us plus 6 for the reduce.  test_abi_host checks the split counts
    against the library's workspace sizes."""
    best, best_us = (0, 1), None
    if M <= 128:
        return best
    KT, mt = (K + 127) // 128, (M + 255) // 256
    for fn in (8, 7, 6, 4, 3, 2):
        tiles = mt * ((N + 32 * fn - 1) // (32 * fn))
        ktile = 0.76 + 0.25 * fn
        for s in range(1, 5):
            per = (KT + s - 1) // s
            if (KT + per - 1) // per != s or (s > 1 and per < 4):
                continue
            full, tail = divmod(tiles * s, 256)
            us = full * (1.3 + per * ktile)
            if tail:
                us += 1.3 + per * ktile * (0.95 + 0.05 * tail / 256)
            if s > 1:
                us += s * M * N * 8 / 6.0e6 + 6.0
            if best_us is None or us < best_us:
                best, best_us = (fn, s), us
    return best


def gemv_splits(M: int, N: int, K: int, int4: bool = False) -> int:
    """K splits of the small-M streaming kernel (M <= 16): among the split
    counts that keep about 256 blocks at most (512 for K < 32 k-tiles) and 8
    (4) k-tiles per split, the one the library's cost model picks: a block
    streams its strip's weight bytes (2 KiB per k-tile, 1 KiB for int4) at
    45 GB/s, and a split costs 3.6 us.  test_abi_host checks it against the
    library's workspace sizes."""
    KT = (K + 127) // 128
    groups = (N // 16) * ((M + 15) // 16)
    target, min_kt = (512, 4) if KT < 32 else (256, 8)
    smax = 1
    while groups * smax < target and smax * 2 <= 8 and KT // (smax * 2) >= min_kt:
        smax *= 2
    strip = KT * (1024 if int4 else 2048)
    s, best = 1, strip / 45e3
    c = 2
    while c <= smax:
        cost = 3.6 + strip / c / 45e3
        if cost < best:
            s, best = c, cost
        c *= 2
    per = (KT + s - 1) // s
    return (KT + per - 1) // per


def w4a16_plan(M: int, N: int, K: int) -> tuple:
    """(fn, splits) of the per-group W4A16 tile kernel (M > 16): 128-row
    blocks of 64 fn columns, the library's cost model in k-tile times of a
    256-column block: rounds of 256 blocks times ceil(KT / s) k-tiles (a
    128-column block's k-tile at 0.6), plus 8 bytes per output and split at
    9 MB per k-tile time; at most 8 splits of 4+ k-tiles."""
    kt = K // 128
    best, best_cost = (4, 1), None
    for fn in (4, 2):
        qn = 64 * fn
        tiles = ((M + 127) // 128) * ((N + qn - 1) // qn)
        ktile = 1.0 if fn == 4 else 0.6
        s = 1
        while s <= 8 and (s == 1 or kt // s >= 4):
            cost = ((tiles * s + 255) // 256) * ((kt + s - 1) // s) * ktile
            if s > 1:
                cost += s * M * N * 8 / 9e6
            if best_cost is None or cost < best_cost:
                best, best_cost = (fn, s), cost
            s += 1
    return best

