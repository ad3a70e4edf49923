"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/bql.h declares, and
reject bad arguments on the host with the documented status before anything
is launched.  None of these calls reaches a kernel: every one fails
validation or is a pure size query, or has M = 0 (a no-op).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_quantized_linear_amd as bql

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bql.h")

OK, ERR_NULL, ERR_DTYPE, ERR_SHAPE, ERR_ALIGN, ERR_WS, ERR_HIP, ERR_ARG = range(8)
A16 = ctypes.c_void_p(0x10000)       # fake, aligned: never dereferenced on these paths
MIS = ctypes.c_void_p(0x10008)       # fake, 8-byte aligned only


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bql_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return bql.lib()


def test_header_declares_the_binding_surface():
    assert header_functions() == sorted(bql.SIGNATURES)


def test_library_exports_every_declared_symbol(L):
    for name in header_functions():
        assert hasattr(L, name), name


def test_abi_version(L):
    assert L.bql_abi_version() == 1


def test_packed_weight_bytes(L):
    # 16 x 128 tiles; K padded up to a multiple of 128
    assert L.bql_packed_weight_bytes(4096, 4096, 1) == 4096 * 4096
    assert L.bql_packed_weight_bytes(4096, 4096, 2) == 4096 * 4096
    assert L.bql_packed_weight_bytes(4096, 4096, 3) == 4096 * 4096 // 2
    assert L.bql_packed_weight_bytes(48, 144, 1) == 3 * 2 * 2048
    assert L.bql_packed_weight_bytes(48, 144, 3) == 3 * 2 * 1024
    assert L.bql_packed_weight_bytes(0, 16, 1) == 0


def test_workspace_sizes_are_monotone_and_cover_aq(L):
    for (M, N, K) in [(1, 4096, 4096), (16, 1024, 1024), (1024, 28672, 4096), (4096, 8192, 28672)]:
        ws = L.bql_fp8_linear_workspace_size(M, N, K)
        assert ws >= 8192 + M * K
        assert L.bql_w8a16_linear_workspace_size(M, N, K) % 256 == 0
        assert L.bql_w4a8_linear_workspace_size(M, N, K) % 256 == 0
    assert L.bql_fp8_linear_workspace_size(0, 16, 16) == 0
    assert L.bql_quantize_workspace_size(123) >= 4096 + 4


def _err(L):
    return L.bql_last_error().decode()


def test_fp8_linear_validation(L):
    f = L.bql_fp8_linear
    ws = L.bql_fp8_linear_workspace_size(4, 64, 64)
    args = dict(a=A16, adt=2, sa=None, w=A16, ws_=A16, pc=0, M=4, N=64, K=64, os_=None,
                y=A16, ydt=2, acc=0, work=A16, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["a"], a["adt"], a["sa"], a["w"], a["ws_"], a["pc"], a["M"], a["N"], a["K"],
                 a["os_"], a["y"], a["ydt"], a["acc"], a["work"], a["wsb"], None)

    assert call(a=None) == ERR_NULL and "a is NULL" in _err(L)
    assert call(w=None) == ERR_NULL
    assert call(y=None) == ERR_NULL
    assert call(ws_=None) == ERR_NULL
    assert call(a=MIS) == ERR_ALIGN
    assert call(N=60) == ERR_SHAPE and "multiples of 16" in _err(L)
    assert call(K=8) == ERR_SHAPE
    assert call(M=-1) == ERR_SHAPE
    assert call(M=(1 << 22) + 1) == ERR_SHAPE
    assert call(adt=5) == ERR_DTYPE
    assert call(ydt=6) == ERR_DTYPE
    assert call(ydt=5) == ERR_DTYPE
    assert call(pc=2) == ERR_ARG
    assert call(acc=2) == ERR_ARG
    assert call(adt=4) == ERR_NULL          # pre-quantized A needs a_scale
    assert call(ydt=4) == ERR_NULL          # fp8 output needs output_scale
    assert call(work=None) == ERR_WS
    assert call(wsb=ws - 1) == ERR_WS
    assert call(work=ctypes.c_void_p(0x10010)) == ERR_ALIGN  # workspace needs 256
    assert call(M=0, wsb=0, work=None) == OK  # no-op


def test_packed_activation_validation(L):
    assert L.bql_fp8_packed_activation_bytes(17, 130) == 2 * 2 * 2048
    assert L.bql_fp8_packed_activation_bytes(0, 128) == 0
    f = L.bql_fp8_pack_activations
    assert f(A16, 32, 120, A16, None) == ERR_SHAPE and "multiple of 16" in _err(L)
    assert f(A16, -1, 128, A16, None) == ERR_SHAPE
    assert f(None, 32, 128, A16, None) == ERR_NULL
    assert f(A16, 32, 128, None, None) == ERR_NULL
    assert f(MIS, 32, 128, A16, None) == ERR_ALIGN
    assert f(None, 0, 128, None, None) == OK  # no-op
    # bql_fp8_linear with BQL_E4M3_TILES: the tile kernels only (M > 16, N >= 16)
    g = L.bql_fp8_linear
    ws = L.bql_fp8_linear_workspace_size(32, 64, 64)

    def call(M=32, N=64, sa=A16):
        return g(A16, 8, sa, A16, A16, 0, M, N, 64, None, A16, 2, 0, A16, ws, None)

    assert call(M=16) == ERR_SHAPE and "M > 16" in _err(L)
    assert call(N=8) == ERR_SHAPE
    assert call(sa=None) == ERR_NULL        # packed codes need a_scale
    assert call(M=0) == OK


def test_fp8_linear_noalloc_validation(L):
    # same checks as bql_fp8_linear, and shapes whose scratch exceeds the
    # library's fixed array are refused before anything is launched
    f = L.bql_fp8_linear_noalloc

    def call(a=A16, adt=2, sa=None, w=A16, sw=A16, pc=0, M=4, N=64, K=64, os_=None, y=A16, ydt=2,
             acc=0):
        return f(a, adt, sa, w, sw, pc, M, N, K, os_, y, ydt, acc, None)

    assert call(a=None) == ERR_NULL
    assert call(y=MIS) == ERR_ALIGN
    assert call(N=60) == ERR_SHAPE
    assert call(adt=5) == ERR_DTYPE
    assert call(acc=3) == ERR_ARG
    assert call(adt=4) == ERR_NULL          # pre-quantized A needs a_scale
    assert call(M=0) == OK                  # no-op
    cap = bql.NOALLOC_SCRATCH_BYTES
    M, N, K = 8192, 4096, 8192              # 64 MiB of packed codes + the quantizer's 8 KiB
    assert L.bql_fp8_linear_workspace_size(M, N, K) > cap
    assert call(M=M, N=N, K=K) == ERR_SHAPE and "noalloc" in _err(L)
    M, N, K = 1024, 28672, 4096
    assert L.bql_fp8_linear_workspace_size(M, N, K) <= cap


def test_quantizer_validation(L):
    q = L.bql_fp8_quantize_dynamic
    assert q(None, 1, 10, A16, None, A16, 8192, None) == ERR_NULL
    assert q(A16, 3, 10, A16, None, A16, 8192, None) == ERR_DTYPE
    assert q(A16, 1, -1, A16, None, A16, 8192, None) == ERR_SHAPE
    assert q(A16, 1, 10, A16, None, None, 0, None) == ERR_WS
    assert q(A16, 1, 10, A16, None, A16, 100, None) == ERR_WS
    assert q(A16, 1, 0, A16, None, A16, 8192, None) == OK
    s = L.bql_fp8_quantize_static
    assert s(A16, 2, 10, None, A16, None) == ERR_NULL
    assert s(A16, 2, 0, A16, A16, None) == OK
    p = L.bql_int8_quantize_per_token
    assert p(A16, 1, 4, 24, A16, A16, None) == ERR_SHAPE
    assert p(A16, 1, 4, 32, A16, None, None) == ERR_NULL
    assert p(A16, 1, 0, 32, A16, A16, None) == OK


def test_w4a8_group_validation(L):
    f = L.bql_w4a8_group_linear
    ws = L.bql_w4a8_linear_workspace_size(4, 64, 256)

    def call(aq=A16, sa=A16, w=A16, sw=A16, M=4, N=64, K=256, g=128, y=A16, ydt=1, work=A16,
             wsb=ws):
        return f(aq, sa, w, sw, M, N, K, g, y, ydt, work, wsb, None)
    assert call(g=64) == ERR_ARG
    assert call(K=272) == ERR_SHAPE                # not a multiple of 128
    assert call(K=128 * 129) == ERR_SHAPE          # above the staged-scale limit
    assert call(ydt=6) == ERR_DTYPE                # no raw int32 output per group
    assert call(sa=None) == ERR_NULL
    assert call(sw=None) == ERR_NULL
    assert call(work=None) == ERR_WS
    assert call(M=0, work=None, wsb=0) == OK
    assert L.bql_packed_weight_bytes(64, 256, 4) == L.bql_packed_weight_bytes(64, 256, 3)
    p = L.bql_prepack_weight
    assert p(A16, 7, 64, 272, 4, A16, 1, A16, A16, None, 0, None) == ERR_SHAPE
    assert p(A16, 7, 64, 256, 4, None, 1, A16, A16, None, 0, None) == ERR_NULL
    assert p(A16, 1, 64, 256, 4, A16, 1, A16, A16, None, 0, None) == ERR_DTYPE


def test_w4a16_group_validation(L):
    f = L.bql_w4a16_group_linear
    ws = L.bql_w4a16_linear_workspace_size(4, 64, 256)

    def call(a=A16, w=A16, s=A16, M=4, N=64, K=256, gs=128, y=A16, ydt=1, work=A16, wsb=ws):
        return f(a, w, s, M, N, K, gs, y, ydt, work, wsb, None)

    assert call(gs=64) == ERR_ARG
    assert call(K=200) == ERR_SHAPE      # a multiple of 16 but not of 128
    assert call(N=60) == ERR_SHAPE
    assert call(ydt=4) == ERR_DTYPE      # no fp8 output
    assert call(ydt=6) == ERR_DTYPE
    assert call(s=None) == ERR_NULL
    assert call(a=MIS) == ERR_ALIGN
    assert call(M=-1) == ERR_SHAPE
    assert call(M=0) == OK
    assert L.bql_w4a16_linear_workspace_size(0, 64, 256) == 0


def test_small_n_shape_rule(L):
    # the fp8 formats take 1 <= N <= 15 (one padded strip); others keep N % 16
    assert L.bql_packed_weight_bytes(8, 4096, 1) == 32 * 2048
    assert L.bql_packed_weight_bytes(1, 48, 2) == 2048
    f = L.bql_fp8_linear
    for N, want in ((8, OK), (1, OK), (15, OK), (24, ERR_SHAPE), (0, ERR_SHAPE)):
        assert f(A16, 2, None, A16, A16, 0, 0, N, 64, None, A16, 2, 0, None, 0, None) == want, N
    assert f(A16, 2, None, A16, A16, 0, 0, 8, 40, None, A16, 2, 0, None, 0, None) == ERR_SHAPE
    s = L.bql_fp8_linear_static
    assert s(A16, 2, A16, A16, A16, 0, 0, 8, 64, None, A16, 2, 0, None, 0, None) == OK
    w = L.bql_w8a16_linear
    assert w(A16, A16, A16, 0, 8, 64, A16, 1, None, 0, None) == ERR_SHAPE
    q = L.bql_w4a8_linear
    assert q(A16, A16, A16, A16, 0, 8, 64, A16, 1, None, 0, None) == ERR_SHAPE
    p = L.bql_prepack_weight
    assert p(A16, 7, 8, 64, 3, A16, 1, A16, A16, None, 0, None) == ERR_SHAPE  # int4 keeps N % 16


def test_fp8_linear_static_validation(L):
    f = L.bql_fp8_linear_static
    ws = L.bql_fp8_linear_workspace_size(4, 64, 64)

    def call(a=A16, adt=2, sc=A16, w=A16, wsc=A16, pc=0, M=4, N=64, K=64, osc=None, y=A16, ydt=2,
             acc=0, work=A16, wsb=ws):
        return f(a, adt, sc, w, wsc, pc, M, N, K, osc, y, ydt, acc, work, wsb, None)
    assert call(sc=None) == ERR_NULL
    assert call(adt=4) == ERR_DTYPE          # pre-quantized input has no static cast
    assert call(N=60) == ERR_SHAPE
    assert call(ydt=4) == ERR_NULL           # fp8 out needs output_scale
    assert call(acc=2) == ERR_ARG
    assert call(work=None) == ERR_WS
    assert call(sc=ctypes.c_void_p(0x10002)) == ERR_ALIGN
    assert call(M=0, work=None, wsb=0) == OK


def test_rmsnorm_quantizer_validation(L):
    i8 = L.bql_rmsnorm_int8_quantize_per_token
    f8 = L.bql_rmsnorm_fp8_quantize_dynamic
    assert L.bql_rmsnorm_quantize_workspace_size(0) == 0
    assert L.bql_rmsnorm_quantize_workspace_size(1024) >= 8 * 1024
    assert L.bql_rmsnorm_quantize_workspace_size(1024) % 256 == 0
    assert i8(A16, A16, 3, 4, 4096, 1e-5, A16, A16, None, None) == ERR_DTYPE
    assert i8(A16, A16, 2, 4, 40, 1e-5, A16, A16, None, None) == ERR_SHAPE
    assert i8(A16, A16, 2, 4, 32768 + 16, 1e-5, A16, A16, None, None) == ERR_SHAPE
    assert i8(A16, A16, 2, 4, 4096, 0.0, A16, A16, None, None) == ERR_ARG
    assert i8(A16, A16, 2, 4, 4096, float("nan"), A16, A16, None, None) == ERR_ARG
    assert i8(A16, A16, 2, 4, 4096, float("inf"), A16, A16, None, None) == ERR_ARG
    assert i8(A16, None, 2, 4, 4096, 1e-5, A16, A16, None, None) == ERR_NULL
    assert i8(A16, MIS, 2, 4, 4096, 1e-5, A16, A16, None, None) == ERR_ALIGN
    assert i8(A16, A16, 2, 4, 4096, 1e-5, A16, None, None, None) == ERR_NULL
    assert i8(A16, A16, 2, 0, 4096, 1e-5, A16, A16, None, None) == OK
    ws = L.bql_rmsnorm_quantize_workspace_size(4)
    assert f8(A16, A16, 2, 4, 4096, 1e-5, A16, None, None, A16, ws, None) == ERR_NULL
    assert f8(A16, A16, 2, 4, 4096, 1e-5, A16, A16, None, None, 0, None) == ERR_WS
    assert f8(A16, A16, 2, 4, 4096, 1e-5, A16, A16, None, A16, ws - 1, None) == ERR_WS
    assert f8(A16, A16, 2, 4, 4096, 1e-5, A16, A16, None, ctypes.c_void_p(0x10010), ws,
              None) == ERR_ALIGN
    assert f8(A16, A16, 2, 4, 4096, -1.0, A16, A16, None, A16, ws, None) == ERR_ARG
    assert f8(A16, A16, 2, 0, 4096, 1e-5, A16, A16, None, None, 0, None) == OK


def test_prepack_validation(L):
    f = L.bql_prepack_weight
    assert f(A16, 2, 64, 60, 1, None, 0, A16, A16, A16, 8192, None) == ERR_SHAPE
    assert f(A16, 5, 64, 64, 1, None, 0, A16, A16, A16, 8192, None) == ERR_DTYPE
    assert f(A16, 2, 64, 64, 9, None, 0, A16, A16, A16, 8192, None) == ERR_ARG
    assert f(A16, 4, 64, 64, 1, None, 0, A16, A16, A16, 8192, None) == ERR_NULL  # codes need scales
    assert f(A16, 2, 64, 64, 3, A16, 1, A16, A16, None, 0, None) == ERR_DTYPE    # int4 needs INT4
    assert f(A16, 7, 64, 64, 3, None, 0, A16, A16, None, 0, None) == ERR_NULL    # int4 needs scales
    assert f(A16, 2, 64, 64, 1, None, 0, A16, A16, None, 0, None) == ERR_WS      # per-tensor amax ws
    assert f(A16, 2, 64, 64, 1, A16, 2, A16, A16, None, 0, None) == ERR_DTYPE    # bf16 scales refused
    u = L.bql_unpack_weight
    assert u(None, 64, 64, 1, A16, None) == ERR_NULL
    assert u(A16, 64, 64, 7, A16, None) == ERR_ARG


def test_w8a16_and_w4a8_validation(L):
    f = L.bql_w8a16_linear
    ws = L.bql_w8a16_linear_workspace_size(1, 64, 64)
    assert f(A16, A16, A16, 1, 64, 64, A16, 4, A16, ws, None) == ERR_DTYPE
    assert f(A16, A16, None, 1, 64, 64, A16, 1, A16, ws, None) == ERR_NULL
    assert f(A16, A16, A16, 0, 64, 64, A16, 1, None, 0, None) == OK
    g = L.bql_w4a8_linear
    ws = L.bql_w4a8_linear_workspace_size(1, 64, 64)
    assert g(A16, A16, A16, A16, 1, 64, 64, A16, 4, A16, ws, None) == ERR_DTYPE
    assert g(A16, None, A16, A16, 1, 64, 64, A16, 1, A16, ws, None) == ERR_NULL
    assert g(A16, A16, A16, A16, 1, 64, 131088, A16, 1, A16, ws, None) == ERR_SHAPE
    # 16 * acc stays inside int32 for K <= 131056 even with -128 codes
    assert g(A16, A16, A16, A16, 1, 64, 131072, A16, 1, A16, ws, None) == ERR_SHAPE
    assert g(A16, None, A16, None, 0, 64, 131056, A16, 6, None, 0, None) == OK
    assert g(A16, None, A16, None, 0, 64, 64, A16, 6, None, 0, None) == OK  # raw int32: scales optional


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        bql.quantize_dynamic(torch.zeros(16, dtype=torch.float16))


def test_exact_tile_plan_mirror(L):
    """The test-side mirror of the exact fp8 kernel's planner gives the split
    count the library sizes its workspace for (shapes where the fast fp8
    kernels do not split, so the fp8 workspace holds the exact path's
    partials only)."""
    from _common import exact_plan
    checked = 0
    for M in (129, 200, 256, 300, 384, 512, 520, 777, 1000, 1024, 1300, 2048, 4096):
        for N in (1040, 2096, 4096, 6144, 8192, 10240, 16352, 28672, 57344):
            for K in (1000, 2000, 4000, 4096, 8192, 14336, 28672):
                if ((M + 127) // 128) * ((N + 127) // 128) <= 256:
                    continue
                ws = L.bql_fp8_linear_workspace_size(M, N, K)
                aq = ((M + 15) // 16) * ((K + 127) // 128) * 2048
                extra = ws - 8192 - (aq + 255) // 256 * 256
                fn, s = exact_plan(M, N, K)
                assert fn != 0
                want = (M * N * 4 * s + 255) // 256 * 256 if s > 1 else 0
                assert extra == want, (M, N, K, fn, s, extra)
                checked += 1
    assert checked > 400


def _split_ws(M, N, K, s):
    KT = (K + 127) // 128
    per = (KT + s - 1) // s
    n = (KT + per - 1) // per
    return (n * M * N * 4 + 255) // 256 * 256 if n > 1 else 0


def test_small_m_split_plan_mirror(L):
    """The test-side mirror of the small-M kernel's split plan gives the
    partial buffers the library sizes its workspaces for (W8A16 and W4A8
    run the small-M kernel at M <= 16)."""
    from _common import gemv_splits
    splits_seen = set()
    for M in (1, 2, 4, 8, 16):
        for N in (16, 256, 1024, 2048, 4096, 6144):
            for K in (128, 1024, 4096, 8192, 16384, 34816, 65536):
                s = gemv_splits(M, N, K)
                assert L.bql_w8a16_linear_workspace_size(M, N, K) == _split_ws(M, N, K, s), (M, N, K, s)
                s4 = gemv_splits(M, N, K, int4=True)
                aq = ((M + 15) // 16) * ((K + 127) // 128) * 2048  # the packed-A region
                got = L.bql_w4a8_linear_workspace_size(M, N, K) - (aq + 255) // 256 * 256
                assert got == _split_ws(M, N, K, s4), (M, N, K, s4)
                splits_seen |= {s, s4}
    assert {1, 2, 4, 8} <= splits_seen


def test_w4a16_tile_plan_mirror(L):
    """The test-side mirror of the per-group W4A16 tile kernel's plan gives
    the split count the library sizes its workspace for, and both block
    widths occur."""
    from _common import w4a16_plan
    widths = set()
    for M in (17, 100, 256, 512, 1000, 1024, 2048, 4096):
        for N in (272, 1040, 2064, 4096, 5120, 6656, 8192):
            for K in (128, 1024, 4096, 5120, 8192, 14336):
                fn, s = w4a16_plan(M, N, K)
                assert L.bql_w4a16_linear_workspace_size(M, N, K) == _split_ws(M, N, K, s), (M, N, K, fn, s)
                widths.add(fn)
    assert widths == {2, 4}

