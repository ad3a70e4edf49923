"""Quantized linear layers for AMD MI355X (gfx950).

A thin ctypes binding over ``libbql.so`` (C ABI in ``include/bql.h``).  This
module only marshals arguments: it takes device pointers and the current
HIP stream from PyTorch tensors, allocates outputs and workspaces with
PyTorch, and calls one library entry point.  Every step of the computation
runs in the library's HIP kernels; there is no fallback of any kind, and
calling a compute function without the built library raises.

Operations (see the header for the exact contracts):
  quantize_dynamic        per-tensor E4M3 with scale = amax / 448
  quantize_static         E4M3 with a given scale
  pack_activations        E4M3 codes into the tile layout fp8_linear reads (M > 16)
  int8_quantize_per_token per-row int8 with scale = amax / 127
  rmsnorm_int8_quantize_per_token   RMSNorm fused with per-row int8
  rmsnorm_fp8_quantize_dynamic      RMSNorm fused with per-tensor E4M3
  prepack_weight          quantize + lay out a weight once after load
  unpack_weight           logical codes back from the packed layout
  fp8_linear              Y = (sA sW[n]) (Aq Wq^T), fp16/bf16/E4M3 output
  fp8_linear_static       the same with a given (static) activation scale
  fp8_linear_noalloc      fp8_linear on the library's own scratch (no workspace)
  w8a16_linear            Y = sW[n] (A Wq^T), fp16 activations
  w4a8_linear             int4 x int8 with int32 accumulation
  w4a8_group_linear       the same with a scale per channel and 128-k group
  w4a16_group_linear      fp16 x int4 weight-only, a scale per channel and 128-k group
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbql.so")

# bql_dtype
F16, BF16, F32, E4M3, I8, I32, INT4, E4M3_TILES = 1, 2, 3, 4, 5, 6, 7, 8
# bql_wfmt
WFMT = {"fp8_tensor": 1, "fp8_channel": 2, "int4_channel": 3, "int4_group": 4}
STATUS = {0: "BQL_OK", 1: "BQL_ERR_NULL", 2: "BQL_ERR_DTYPE", 3: "BQL_ERR_SHAPE",
          4: "BQL_ERR_ALIGN", 5: "BQL_ERR_WORKSPACE", 6: "BQL_ERR_HIP", 7: "BQL_ERR_ARG"}

_TORCH_TO_BQL = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32,
                 torch.uint8: E4M3, torch.float8_e4m3fn: E4M3, torch.int8: I8, torch.int32: I32}


class BQLError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {message}")
        self.status = status


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SZ = ctypes.c_size_t

# name -> (restype, argtypes): the complete exported surface of include/bql.h
SIGNATURES = {
    "bql_abi_version": (_I, []),
    "bql_last_error": (ctypes.c_char_p, []),
    "bql_quantize_workspace_size": (_SZ, [_I64]),
    "bql_fp8_quantize_dynamic": (_I, [_P, _I, _I64, _P, _P, _P, _SZ, _P]),
    "bql_fp8_quantize_static": (_I, [_P, _I, _I64, _P, _P, _P]),
    "bql_fp8_packed_activation_bytes": (_SZ, [_I64, _I64]),
    "bql_fp8_pack_activations": (_I, [_P, _I64, _I64, _P, _P]),
    "bql_int8_quantize_per_token": (_I, [_P, _I, _I64, _I64, _P, _P, _P]),
    "bql_rmsnorm_quantize_workspace_size": (_SZ, [_I64]),
    "bql_rmsnorm_int8_quantize_per_token": (_I, [_P, _P, _I, _I64, _I64, ctypes.c_float, _P, _P,
                                                 _P, _P]),
    "bql_rmsnorm_fp8_quantize_dynamic": (_I, [_P, _P, _I, _I64, _I64, ctypes.c_float, _P, _P, _P,
                                              _P, _SZ, _P]),
    "bql_packed_weight_bytes": (_SZ, [_I64, _I64, _I]),
    "bql_prepack_workspace_size": (_SZ, [_I64, _I64, _I]),
    "bql_prepack_weight": (_I, [_P, _I, _I64, _I64, _I, _P, _I, _P, _P, _P, _SZ, _P]),
    "bql_unpack_weight": (_I, [_P, _I64, _I64, _I, _P, _P]),
    "bql_fp8_linear_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "bql_fp8_linear": (_I, [_P, _I, _P, _P, _P, _I, _I64, _I64, _I64, _P, _P, _I, _I, _P, _SZ, _P]),
    "bql_fp8_linear_static": (_I, [_P, _I, _P, _P, _P, _I, _I64, _I64, _I64, _P, _P, _I, _I, _P, _SZ,
                                   _P]),
    "bql_fp8_linear_noalloc": (_I, [_P, _I, _P, _P, _P, _I, _I64, _I64, _I64, _P, _P, _I, _I, _P]),
    "bql_w8a16_linear_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "bql_w8a16_linear": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _I, _P, _SZ, _P]),
    "bql_w4a8_linear_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "bql_w4a8_linear": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P, _SZ, _P]),
    "bql_w4a8_group_linear": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I, _P, _SZ, _P]),
    "bql_w4a16_linear_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "bql_w4a16_group_linear": (_I, [_P, _P, _P, _I64, _I64, _I64, _I64, _P, _I, _P, _SZ, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python bit_quantized_linear_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        if L.bql_abi_version() != 1:
            raise ImportError("libbql.so ABI version mismatch")
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise BQLError(fn, status, lib().bql_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must be on a HIP device")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _workspace(nbytes: int, dev: torch.device, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    return ws, ws.numel() * ws.element_size()


# ---------------------------------------------------------------- quantizers

def quantize_dynamic(x: torch.Tensor, ws: Optional[torch.Tensor] = None):
    """Per-tensor E4M3: returns (codes uint8 shaped like x, scale fp32 [1])."""
    _need_cuda(x)
    L = lib()
    xq = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scale = torch.empty(1, dtype=torch.float32, device=x.device)
    ws, nb = _workspace(L.bql_quantize_workspace_size(x.numel()), x.device, ws)
    _check("bql_fp8_quantize_dynamic",
           L.bql_fp8_quantize_dynamic(_ptr(x), _TORCH_TO_BQL[x.dtype], x.numel(), _ptr(xq),
                                      _ptr(scale), _ptr(ws), nb, _stream(x.device)))
    return xq, scale


@dataclass
class PackedActivations:
    """E4M3 activation codes [M,K] in the library's operand-tile layout."""
    packed: torch.Tensor   # uint8, private tile layout
    M: int
    K: int


def pack_activations(codes: torch.Tensor) -> PackedActivations:
    """Row-major E4M3 codes [M,K] (uint8 or float8_e4m3fn) into the layout
    the large-M fp8 GEMMs read, for fp8_linear calls that should not repack
    A each time (M > 16)."""
    _need_cuda(codes)
    L = lib()
    M, K = codes.shape
    packed = torch.empty(max(16, L.bql_fp8_packed_activation_bytes(M, K)), dtype=torch.uint8,
                         device=codes.device)
    _check("bql_fp8_pack_activations",
           L.bql_fp8_pack_activations(_ptr(codes), M, K, _ptr(packed), _stream(codes.device)))
    return PackedActivations(packed, M, K)


def quantize_static(x: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    _need_cuda(x, scale)
    L = lib()
    xq = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check("bql_fp8_quantize_static",
           L.bql_fp8_quantize_static(_ptr(x), _TORCH_TO_BQL[x.dtype], x.numel(), _ptr(scale),
                                     _ptr(xq), _stream(x.device)))
    return xq


def int8_quantize_per_token(x: torch.Tensor):
    """Per-row symmetric int8: returns (codes int8 [M,K], scales fp32 [M])."""
    _need_cuda(x)
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    sc = torch.empty(M, dtype=torch.float32, device=x.device)
    _check("bql_int8_quantize_per_token",
           lib().bql_int8_quantize_per_token(_ptr(x), _TORCH_TO_BQL[x.dtype], M, K, _ptr(xq),
                                             _ptr(sc), _stream(x.device)))
    return xq, sc


def _rmsnorm_args(x: torch.Tensor, g: torch.Tensor):
    _need_cuda(x, g)
    if x.dim() != 2 or g.shape != (x.shape[1],) or g.dtype != x.dtype:
        raise ValueError("x must be [M,K] and g [K] of the same dtype")
    return x.shape


def rmsnorm_int8_quantize_per_token(x: torch.Tensor, g: torch.Tensor, eps: float,
                                    inv_rms: bool = False):
    """RMSNorm(x) * g, then per-row int8: returns (codes int8 [M,K],
    scales fp32 [M], inv_rms fp32 [M] or None)."""
    M, K = _rmsnorm_args(x, g)
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    sc = torch.empty(M, dtype=torch.float32, device=x.device)
    r = torch.empty(M, dtype=torch.float32, device=x.device) if inv_rms else None
    _check("bql_rmsnorm_int8_quantize_per_token",
           lib().bql_rmsnorm_int8_quantize_per_token(_ptr(x), _ptr(g), _TORCH_TO_BQL[x.dtype], M, K,
                                                     float(eps), _ptr(xq), _ptr(sc), _ptr(r),
                                                     _stream(x.device)))
    return xq, sc, r


def rmsnorm_fp8_quantize_dynamic(x: torch.Tensor, g: torch.Tensor, eps: float,
                                 inv_rms: bool = False, ws: Optional[torch.Tensor] = None):
    """RMSNorm(x) * g, then per-tensor E4M3: returns (codes uint8 [M,K],
    scale fp32 [1], inv_rms fp32 [M] or None)."""
    M, K = _rmsnorm_args(x, g)
    L = lib()
    xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    scale = torch.empty(1, dtype=torch.float32, device=x.device)
    r = torch.empty(M, dtype=torch.float32, device=x.device) if inv_rms else None
    ws, nb = _workspace(L.bql_rmsnorm_quantize_workspace_size(M), x.device, ws)
    _check("bql_rmsnorm_fp8_quantize_dynamic",
           L.bql_rmsnorm_fp8_quantize_dynamic(_ptr(x), _ptr(g), _TORCH_TO_BQL[x.dtype], M, K,
                                              float(eps), _ptr(xq), _ptr(scale), _ptr(r), _ptr(ws),
                                              nb, _stream(x.device)))
    return xq, scale, r


# ------------------------------------------------------------------- weights

@dataclass
class PackedWeight:
    packed: torch.Tensor   # uint8, private tile layout
    scales: torch.Tensor   # fp32, [1] or [N] in logical channel order; int4_group [K/128 * N]
    N: int
    K: int
    fmt: str

    @property
    def per_channel(self) -> bool:
        return self.fmt != "fp8_tensor"


def packed_weight_bytes(N: int, K: int, fmt: str) -> int:
    return lib().bql_packed_weight_bytes(N, K, WFMT[fmt])


def prepack_weight(w: torch.Tensor, fmt: str = "fp8_tensor", scales: Optional[torch.Tensor] = None,
                   K: Optional[int] = None) -> PackedWeight:
    """Quantize (when w is fp16/bf16) and pack an [N,K] weight.

    w: fp16/bf16 [N,K]; or E4M3 codes (uint8 / float8_e4m3fn) [N,K] with
    `scales`; or, for fmt="int4_channel" / "int4_group", logical int4 bytes uint8 [N,K/2]
    (int4_group: `scales` [N, K/128], stored group-major [K/128, N] in the result)
    with `scales` (pass K when w is flattened)."""
    _need_cuda(w, scales)
    L = lib()
    if fmt in ("int4_channel", "int4_group"):
        N = w.shape[0]
        K = K if K is not None else 2 * w.shape[1]
        wdt = INT4
    else:
        N, K = w.shape
        wdt = _TORCH_TO_BQL[w.dtype]
    packed = torch.empty(L.bql_packed_weight_bytes(N, K, WFMT[fmt]), dtype=torch.uint8, device=w.device)
    nsc = 1 if fmt == "fp8_tensor" else (N * (K // 128) if fmt == "int4_group" else N)
    sc = torch.empty(nsc, dtype=torch.float32, device=w.device)
    ws, nb = _workspace(L.bql_prepack_workspace_size(N, K, WFMT[fmt]), w.device, None)
    sdt = 0 if scales is None else _TORCH_TO_BQL[scales.dtype]
    _check("bql_prepack_weight",
           L.bql_prepack_weight(_ptr(w), wdt, N, K, WFMT[fmt], _ptr(scales), sdt, _ptr(packed),
                                _ptr(sc), _ptr(ws), nb, _stream(w.device)))
    return PackedWeight(packed, sc, N, K, fmt)


def unpack_weight(pw: PackedWeight) -> torch.Tensor:
    """Logical codes: uint8 [N,K] (fp8) or logical int4 bytes uint8 [N,K/2]."""
    shape = (pw.N, pw.K // 2) if pw.fmt in ("int4_channel", "int4_group") else (pw.N, pw.K)
    out = torch.empty(shape, dtype=torch.uint8, device=pw.packed.device)
    _check("bql_unpack_weight",
           lib().bql_unpack_weight(_ptr(pw.packed), pw.N, pw.K, WFMT[pw.fmt], _ptr(out),
                                   _stream(pw.packed.device)))
    return out


# ------------------------------------------------------------------- linears

def fp8_linear_workspace_size(M: int, N: int, K: int) -> int:
    return lib().bql_fp8_linear_workspace_size(M, N, K)


def fp8_linear(a: torch.Tensor, pw: PackedWeight, a_scale: Optional[torch.Tensor] = None,
               out_dtype: torch.dtype = torch.bfloat16, output_scale: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
               fast_accum: bool = False) -> torch.Tensor:
    """Y = (sA sW[n]) (Aq Wq^T).

    a fp16/bf16 [M,K]: quantized dynamically per tensor (the scale used is
    written to `a_scale` if given, an fp32 [1] tensor).  a uint8 /
    float8_e4m3fn codes: pre-quantized, `a_scale` required; a
    PackedActivations (M > 16): the same codes already packed.
    out_dtype float16 / bfloat16 / float32, or float8_e4m3fn/uint8 with
    `output_scale`.  fast_accum=True uses the fp8 matrix cores' own
    accumulation (BQL_ACCUM_FAST) instead of exact products summed in fp32."""
    if isinstance(a, PackedActivations):
        M, K, adt, a = a.M, a.K, E4M3_TILES, a.packed
    else:
        M, K = a.shape
        adt = _TORCH_TO_BQL[a.dtype]
    _need_cuda(a, a_scale, output_scale, out, ws)
    L = lib()
    N = pw.N
    ydt = _TORCH_TO_BQL[out_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=torch.uint8 if ydt == E4M3 else out_dtype, device=a.device)
    ws, nb = _workspace(L.bql_fp8_linear_workspace_size(M, N, K), a.device, ws)
    _check("bql_fp8_linear",
           L.bql_fp8_linear(_ptr(a), adt, _ptr(a_scale), _ptr(pw.packed),
                            _ptr(pw.scales), int(pw.per_channel), M, N, K, _ptr(output_scale),
                            _ptr(out), ydt, int(bool(fast_accum)), _ptr(ws), nb, _stream(a.device)))
    return out


def fp8_linear_static(a: torch.Tensor, pw: PackedWeight, a_scale: torch.Tensor,
                      out_dtype: torch.dtype = torch.bfloat16,
                      output_scale: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                      fast_accum: bool = False) -> torch.Tensor:
    """Y = (sA sW[n]) (Aq Wq^T) with Aq = E4M3(A / a_scale) for a given fp32 [1]
    activation scale (static input_scale, or one kept from an earlier call)."""
    _need_cuda(a, a_scale, output_scale, out, ws)
    L = lib()
    M, K = a.shape
    N = pw.N
    ydt = _TORCH_TO_BQL[out_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=torch.uint8 if ydt == E4M3 else out_dtype, device=a.device)
    ws, nb = _workspace(L.bql_fp8_linear_workspace_size(M, N, K), a.device, ws)
    _check("bql_fp8_linear_static",
           L.bql_fp8_linear_static(_ptr(a), _TORCH_TO_BQL[a.dtype], _ptr(a_scale), _ptr(pw.packed),
                                   _ptr(pw.scales), int(pw.per_channel), M, N, K,
                                   _ptr(output_scale), _ptr(out), ydt, int(bool(fast_accum)),
                                   _ptr(ws), nb, _stream(a.device)))
    return out


# scratch the library holds for fp8_linear_noalloc (BQL_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


def fp8_linear_noalloc(a: torch.Tensor, pw: PackedWeight, a_scale: Optional[torch.Tensor] = None,
                       out_dtype: torch.dtype = torch.bfloat16,
                       output_scale: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, fast_accum: bool = False) -> torch.Tensor:
    """fp8_linear on the library's own per-GPU scratch: no workspace argument
    and no allocation inside the call (`out` may be given so that the call
    allocates nothing at all).  Calls overlapping on one GPU race.  `a` as
    for fp8_linear, PackedActivations included."""
    if isinstance(a, PackedActivations):
        M, K, adt, a = a.M, a.K, E4M3_TILES, a.packed
    else:
        M, K = a.shape
        adt = _TORCH_TO_BQL[a.dtype]
    _need_cuda(a, a_scale, output_scale, out)
    L = lib()
    N = pw.N
    ydt = _TORCH_TO_BQL[out_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=torch.uint8 if ydt == E4M3 else out_dtype, device=a.device)
    _check("bql_fp8_linear_noalloc",
           L.bql_fp8_linear_noalloc(_ptr(a), adt, _ptr(a_scale), _ptr(pw.packed),
                                    _ptr(pw.scales), int(pw.per_channel), M, N, K,
                                    _ptr(output_scale), _ptr(out), ydt, int(bool(fast_accum)),
                                    _stream(a.device)))
    return out


def w8a16_linear(a: torch.Tensor, pw: PackedWeight, out_dtype: torch.dtype = torch.float16,
                 out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need_cuda(a, out, ws)
    L = lib()
    M, K = a.shape
    N = pw.N
    if pw.fmt != "fp8_channel":
        raise ValueError("w8a16_linear takes an fp8_channel weight")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    ws, nb = _workspace(L.bql_w8a16_linear_workspace_size(M, N, K), a.device, ws)
    _check("bql_w8a16_linear",
           L.bql_w8a16_linear(_ptr(a), _ptr(pw.packed), _ptr(pw.scales), M, N, K, _ptr(out),
                              _TORCH_TO_BQL[out_dtype], _ptr(ws), nb, _stream(a.device)))
    return out


def w4a8_group_linear(aq: torch.Tensor, a_scales: torch.Tensor, pw: PackedWeight,
                      out_dtype: torch.dtype = torch.float16, out: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int8 [M,K] activations (per-row scales) x int4 weight with a scale per
    output channel and 128-k group (prepacked as "int4_group")."""
    _need_cuda(aq, a_scales, out, ws)
    L = lib()
    M, K = aq.shape
    N = pw.N
    if pw.fmt != "int4_group":
        raise ValueError("w4a8_group_linear takes an int4_group weight")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=aq.device)
    ws, nb = _workspace(L.bql_w4a8_linear_workspace_size(M, N, K), aq.device, ws)
    _check("bql_w4a8_group_linear",
           L.bql_w4a8_group_linear(_ptr(aq), _ptr(a_scales), _ptr(pw.packed), _ptr(pw.scales), M, N,
                                   K, 128, _ptr(out), _TORCH_TO_BQL[out_dtype], _ptr(ws), nb,
                                   _stream(aq.device)))
    return out


def w4a16_group_linear(a: torch.Tensor, pw: PackedWeight, out_dtype: torch.dtype = torch.float16,
                       out: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp16 [M,K] activations x int4 weight with a scale per output channel
    and 128-k group (prepacked as "int4_group"), weight-only."""
    _need_cuda(a, out, ws)
    L = lib()
    M, K = a.shape
    N = pw.N
    if pw.fmt != "int4_group":
        raise ValueError("w4a16_group_linear takes an int4_group weight")
    if a.dtype != torch.float16:
        raise ValueError("w4a16_group_linear takes fp16 activations")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    ws, nb = _workspace(L.bql_w4a16_linear_workspace_size(M, N, K), a.device, ws)
    _check("bql_w4a16_group_linear",
           L.bql_w4a16_group_linear(_ptr(a), _ptr(pw.packed), _ptr(pw.scales), M, N, K, 128, _ptr(out),
                                    _TORCH_TO_BQL[out_dtype], _ptr(ws), nb, _stream(a.device)))
    return out


def w4a8_linear(aq: torch.Tensor, a_scales: Optional[torch.Tensor], pw: PackedWeight,
                out_dtype: torch.dtype = torch.float16, out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int8 [M,K] activations (per-row scales) x int4 weight; out_dtype
    float16 / bfloat16, or int32 for the raw accumulator."""
    _need_cuda(aq, a_scales, out, ws)
    L = lib()
    M, K = aq.shape
    N = pw.N
    if pw.fmt != "int4_channel":
        raise ValueError("w4a8_linear takes an int4_channel weight")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=aq.device)
    ws, nb = _workspace(L.bql_w4a8_linear_workspace_size(M, N, K), aq.device, ws)
    _check("bql_w4a8_linear",
           L.bql_w4a8_linear(_ptr(aq), _ptr(a_scales), _ptr(pw.packed), _ptr(pw.scales), M, N, K,
                             _ptr(out), _TORCH_TO_BQL[out_dtype], _ptr(ws), nb, _stream(aq.device)))
    return out
