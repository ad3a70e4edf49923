"""CPU oracle for the quantized-linear hot path (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
import this package.  The product library never does, and shares no code,
header, table or helper with it.

This module is a thin numpy/ctypes wrapper around ``oracle.c`` (plain C,
fp64 / exact integer arithmetic); every function here names the passage of
the pages it follows in the C source.  Inputs are numpy arrays; 16-bit float
inputs are passed as their raw uint16 bit patterns plus a dtype tag, so that
the oracle decodes them itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F16, BF16, F32 = 1, 2, 3
DTYPE_TAG = {"f16": F16, "bf16": BF16, "f32": F32}

GCC_FLAGS = ["-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
             "-fexcess-precision=standard", "-shared", "-fPIC", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so beside it (gcc, no GPU needed)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float


def _declare(L):
    L.bqo_threads.restype = ctypes.c_int
    L.bqo_threads.argtypes = []
    L.bqo_e4m3_decode.restype = ctypes.c_double
    L.bqo_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.bqo_e4m3_encode.restype = ctypes.c_uint8
    L.bqo_e4m3_encode.argtypes = [ctypes.c_double]
    L.bqo_f16_to_f32.restype = ctypes.c_float
    L.bqo_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.bqo_bf16_to_f32.restype = ctypes.c_float
    L.bqo_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.bqo_decode_input.argtypes = [_P, ctypes.c_int, _I64, _P]
    L.bqo_quant_per_tensor.argtypes = [_P, _I64, _P, _P]
    L.bqo_quant_per_row.argtypes = [_P, _I64, _I64, _P, _P]
    L.bqo_quant_with_scales.argtypes = [_P, _I64, _I64, _P, _I64, _P]
    L.bqo_int8_quant_per_token.argtypes = [_P, _I64, _I64, _P, _P]
    L.bqo_unpack_int4.argtypes = [_P, _I64, _I64, _P]
    L.bqo_fp8_acc.argtypes = [_P, _P, _I64, _I64, _I64, _P, _I64, _P]
    L.bqo_fp8_linear.argtypes = [_P, _F, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P, _I64, _P]
    L.bqo_fp8_output.argtypes = [_P, _I64, _F, _P]
    L.bqo_w8a16_linear.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P, _I64, _P]
    L.bqo_w4a8_acc.argtypes = [_P, _P, _I64, _I64, _I64, _P, _I64, _P]
    L.bqo_w4a8_linear.argtypes = [_P, _P, _P, _I64, _P, _I64, _P]
    L.bqo_w4a8_group_linear.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I64, _P]
    L.bqo_w4a16_group_linear.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _P, _I64, _P]
    L.bqo_rms_sumsq.restype = ctypes.c_double
    L.bqo_rms_sumsq.argtypes = [_P, _I64]
    L.bqo_rms_inv.restype = ctypes.c_float
    L.bqo_rms_inv.argtypes = [ctypes.c_double, _I64, _F]
    L.bqo_rmsnorm_apply.argtypes = [_P, _P, _P, _I64, _I64, _P]
    L.bqo_rmsnorm.argtypes = [_P, _P, _I64, _I64, _F, _P, _P]
    for fn in ("bqo_decode_input", "bqo_quant_per_tensor", "bqo_quant_per_row",
               "bqo_quant_with_scales", "bqo_int8_quant_per_token", "bqo_unpack_int4",
               "bqo_fp8_acc", "bqo_fp8_linear", "bqo_fp8_output", "bqo_w8a16_linear",
               "bqo_w4a8_acc", "bqo_w4a8_linear", "bqo_rmsnorm_apply", "bqo_rmsnorm",
               "bqo_w4a8_group_linear", "bqo_w4a16_group_linear"):
        getattr(L, fn).restype = None


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _rows(rows, M):
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < M)
    return rows


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().bqo_threads())


# ------------------------------------------------------------------ scalars

def e4m3_decode(code: int) -> float:
    return lib().bqo_e4m3_decode(int(code) & 0xFF)


def e4m3_encode(v: float) -> int:
    return int(lib().bqo_e4m3_encode(float(v)))


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    enc = lib().bqo_e4m3_encode
    flat = np.asarray(v, dtype=np.float64).ravel()
    return np.array([enc(float(x)) for x in flat], dtype=np.uint8).reshape(np.shape(v))


def e4m3_decode_table() -> np.ndarray:
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


# ------------------------------------------------------------------ inputs

def decode_input(bits: np.ndarray, dtype: str) -> np.ndarray:
    """fp16/bf16 bit patterns (uint16) or fp32 values -> fp32 values."""
    tag = DTYPE_TAG[dtype]
    src = np.ascontiguousarray(bits, dtype=np.float32 if tag == F32 else np.uint16)
    out = np.empty(src.shape, dtype=np.float32)
    lib().bqo_decode_input(_ptr(src), tag, src.size, _ptr(out))
    return out


# ------------------------------------------------------------ quantizers

def quant_per_tensor(x: np.ndarray):
    """Dynamic per-tensor E4M3: returns (codes uint8, scale float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.empty(x.shape, dtype=np.uint8)
    s = np.zeros(1, dtype=np.float32)
    lib().bqo_quant_per_tensor(_ptr(x), x.size, _ptr(q), _ptr(s))
    return q, np.float32(s[0])


def quant_per_row(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    q = np.empty(x.shape, dtype=np.uint8)
    s = np.empty(rows, dtype=np.float32)
    lib().bqo_quant_per_row(_ptr(x), rows, cols, _ptr(q), _ptr(s))
    return q, s


def quant_with_scales(x: np.ndarray, scales: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    scales = np.ascontiguousarray(scales, dtype=np.float32).ravel()
    rows, cols = x.shape
    assert scales.size in (1, rows)
    q = np.empty(x.shape, dtype=np.uint8)
    lib().bqo_quant_with_scales(_ptr(x), rows, cols, _ptr(scales), scales.size, _ptr(q))
    return q


def int8_quant_per_token(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    lib().bqo_int8_quant_per_token(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def unpack_int4(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    assert packed.size == N * K // 2
    w = np.empty((N, K), dtype=np.int8)
    lib().bqo_unpack_int4(_ptr(packed), N, K, _ptr(w))
    return w


# ---------------------------------------------------------------- linears

def fp8_acc(aq, wq, rows=None) -> np.ndarray:
    aq = np.ascontiguousarray(aq, dtype=np.uint8)
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    M, K = aq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K
    r = _rows(rows, M)
    out = np.empty((r.size, N), dtype=np.float64)
    lib().bqo_fp8_acc(_ptr(aq), _ptr(wq), M, N, K, _ptr(r), r.size, _ptr(out))
    return out


def fp8_linear(aq, sa, wq, sw, rows=None) -> np.ndarray:
    """Y = (sA * sW[n]) * (Aq . Wq^T) in fp64 (exact accumulate)."""
    aq = np.ascontiguousarray(aq, dtype=np.uint8)
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    sw = np.ascontiguousarray(np.atleast_1d(sw), dtype=np.float32)
    M, K = aq.shape
    N = wq.shape[0]
    per_channel = 1 if sw.size == N and N != 1 else 0
    if sw.size not in (1, N):
        raise ValueError("weight scale must have 1 or N entries")
    r = _rows(rows, M)
    y = np.empty((r.size, N), dtype=np.float64)
    lib().bqo_fp8_linear(_ptr(aq), float(sa), _ptr(wq), _ptr(sw), per_channel,
                         M, N, K, _ptr(r), r.size, _ptr(y))
    return y


def fp8_output(y: np.ndarray, output_scale: float) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64)
    c = np.empty(y.shape, dtype=np.uint8)
    lib().bqo_fp8_output(_ptr(y), y.size, float(output_scale), _ptr(c))
    return c


def w8a16_linear(a, wq, sw, rows=None) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    sw = np.ascontiguousarray(sw, dtype=np.float32).ravel()
    M, K = a.shape
    N = wq.shape[0]
    assert sw.size == N
    r = _rows(rows, M)
    y = np.empty((r.size, N), dtype=np.float64)
    lib().bqo_w8a16_linear(_ptr(a), _ptr(wq), _ptr(sw), M, N, K, _ptr(r), r.size, _ptr(y))
    return y


def w4a8_acc(aq, w4, rows=None) -> np.ndarray:
    aq = np.ascontiguousarray(aq, dtype=np.int8)
    w4 = np.ascontiguousarray(w4, dtype=np.int8)
    M, K = aq.shape
    N = w4.shape[0]
    r = _rows(rows, M)
    acc = np.empty((r.size, N), dtype=np.int64)
    lib().bqo_w4a8_acc(_ptr(aq), _ptr(w4), M, N, K, _ptr(r), r.size, _ptr(acc))
    if acc.size and (acc.max() > 2**31 - 1 or acc.min() < -(2**31)):
        raise OverflowError("W4A8 accumulator does not fit int32")
    return acc


def w4a8_linear(acc, sa, sw, rows=None) -> np.ndarray:
    acc = np.ascontiguousarray(acc, dtype=np.int64)
    sa = np.ascontiguousarray(sa, dtype=np.float32).ravel()
    sw = np.ascontiguousarray(sw, dtype=np.float32).ravel()
    nr, N = acc.shape
    r = _rows(rows, sa.size)
    assert r.size == nr
    y = np.empty((nr, N), dtype=np.float64)
    lib().bqo_w4a8_linear(_ptr(acc), _ptr(sa), _ptr(sw), N, _ptr(r), nr, _ptr(y))
    return y


# ------------------------------------------------- RMSNorm ahead of quant

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float):
    """RMSNorm in the precision the fused quantizers define (oracle.c):
    returns (y float32 [M,K], r float32 [M])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32).ravel()
    M, K = x.shape
    assert g.size == K
    y = np.empty((M, K), dtype=np.float32)
    r = np.empty(M, dtype=np.float32)
    lib().bqo_rmsnorm(_ptr(x), _ptr(g), M, K, float(eps), _ptr(y), _ptr(r))
    return y, r


def rmsnorm_apply(x: np.ndarray, g: np.ndarray, r: np.ndarray) -> np.ndarray:
    """y = fp32(fp32(x * r[m]) * g[k]) for given per-row r."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32).ravel()
    r = np.ascontiguousarray(r, dtype=np.float32).ravel()
    M, K = x.shape
    assert g.size == K and r.size == M
    y = np.empty((M, K), dtype=np.float32)
    lib().bqo_rmsnorm_apply(_ptr(x), _ptr(g), _ptr(r), M, K, _ptr(y))
    return y


def rms_sumsq(x: np.ndarray) -> np.ndarray:
    """Per-row fp64 sum of squares, in k order."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    L = lib()
    return np.array([L.bqo_rms_sumsq(_ptr(x[m]), K) for m in range(M)], dtype=np.float64)


def rms_inv(sumsq: float, K: int, eps: float) -> np.float32:
    return np.float32(lib().bqo_rms_inv(float(sumsq), int(K), float(eps)))


def rms_inv_candidates(x: np.ndarray, eps: float):
    """Every fp32 r[m] the definition admits.

    The definition sums the squares in fp64 without fixing the order, so a
    sum taken in another order differs from the exact sum by at most
    (K - 1) * 2^-53 of itself (all terms are non-negative).  The fp64 chain
    that follows is monotone in the sum, so the admissible r are the fp32
    values between the chain at the two ends of that interval (widened for
    the oracle's own summation error and the chain's roundings).  Returns
    (r_lo, r_hi) float32 [M]; they differ only for rows whose exact r lies
    next to an fp32 rounding boundary, and then by one ulp."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    delta = (2.0 * K + 16.0) * 2.0 ** -53
    ss = rms_sumsq(x)
    lo = np.array([rms_inv(s * (1.0 + delta), K, eps) for s in ss], dtype=np.float32)
    hi = np.array([rms_inv(s * (1.0 - delta), K, eps) for s in ss], dtype=np.float32)
    assert np.all(lo <= hi)
    assert np.all((hi == lo) | (hi == np.nextafter(lo, np.float32(np.inf)))), \
        "more than two admissible r values"
    return lo, hi


def rmsnorm_int8_per_token(x: np.ndarray, g: np.ndarray, eps: float, r=None):
    """RMSNorm then per-token int8: returns (codes int8, scales float32 [M], r).
    r (optional) picks one admissible r per row (see rms_inv_candidates)."""
    if r is None:
        y, r = rmsnorm(x, g, eps)
    else:
        y = rmsnorm_apply(x, g, r)
    q, s = int8_quant_per_token(y)
    return q, s, r


def rmsnorm_fp8_per_tensor(x: np.ndarray, g: np.ndarray, eps: float, r=None):
    """RMSNorm then dynamic per-tensor E4M3: returns (codes uint8, scale, r)."""
    if r is None:
        y, r = rmsnorm(x, g, eps)
    else:
        y = rmsnorm_apply(x, g, r)
    q, s = quant_per_tensor(y)
    return q, s, r


def w4a8_group_linear(aq, sa, w4, sw, group=128, rows=None) -> np.ndarray:
    """Per-group W4A8 (QQQ issue #15 "qqq-g128", read as one scale per
    output channel and 128-k group): Y = sA[m] * sum_g sW[n,g] * acc_g[m,n],
    acc_g the exact integer sum over group g; fp64.  sw: [N, G]."""
    aq = np.ascontiguousarray(aq, dtype=np.int8)
    w4 = np.ascontiguousarray(w4, dtype=np.int8)
    sa = np.ascontiguousarray(sa, dtype=np.float32).ravel()
    M, K = aq.shape
    N = w4.shape[0]
    G = (K + group - 1) // group
    sw = np.ascontiguousarray(sw, dtype=np.float32).reshape(N, G)
    r = _rows(rows, M)
    y = np.empty((r.size, N), dtype=np.float64)
    lib().bqo_w4a8_group_linear(_ptr(aq), _ptr(sa), _ptr(w4), _ptr(sw), M, N, K, group, _ptr(r),
                                r.size, _ptr(y))
    return y


def w4a16_group_linear(a, w4, sw, group=128, rows=None) -> np.ndarray:
    """Per-group weight-only int4 (QQQ issue #15 "awq-g128" / "marlin-g128",
    read as one scale per output channel and 128-k group, no zero point):
    Y = sum_g sW[n,g] * sum_{k in g} A[m,k] * W4[n,k], fp64.  a: fp32 values
    of the fp16 activations [M, K]; w4: int values [N, K]; sw: [N, G]."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    w4 = np.ascontiguousarray(w4, dtype=np.int8)
    M, K = a.shape
    N = w4.shape[0]
    G = (K + group - 1) // group
    sw = np.ascontiguousarray(sw, dtype=np.float32).reshape(N, G)
    r = _rows(rows, M)
    y = np.empty((r.size, N), dtype=np.float64)
    lib().bqo_w4a16_group_linear(_ptr(a), _ptr(w4), _ptr(sw), M, N, K, group, _ptr(r), r.size,
                                 _ptr(y))
    return y


def within_tolerance(got: np.ndarray, ref: np.ndarray, rel: float = 5e-3, floor: float = 1e-2):
    """The float-output bar: |got - ref| <= rel * (|ref| + floor * max|ref|).

    Returns (ok, worst_ratio) where worst_ratio is max |d| / bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = rel * (np.abs(ref) + floor * (np.abs(ref).max() if ref.size else 0.0))
    d = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, d / bound, np.where(d > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(np.all(d <= bound)), worst
