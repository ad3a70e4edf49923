"""Captured HIP graphs of the linears replay to the eager result.

Every path is captured once (small-M fused and split-K, the tiled kernel,
exact and fast accumulation, W8A16, W4A8, the static-scale linear, the
small-N linear, the fused RMSNorm quantizers, per-group W4A8, pre-quantized
A read row-major by the k-split kernel, pre-packed A into the exact tile
kernel with K split) and replayed
several times with eager work and synchronizations in between; each replay
must equal the eager output bit for bit (all kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from _common import DEV, dev, dev16

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu


def _replays_match(run, out, noise):
    run()
    torch.cuda.synchronize()
    want = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up off the capture stream, as torch recommends
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(3):
        out.zero_()
        noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), want.view(torch.uint8))


@pytest.mark.parametrize("fast", [False, True])
# (1024, 4096, 4096) and (300, 2048, 4096): the exact tile kernel with eight
# waves, the latter with K split; (520, 4208, 8000): four waves, K split
# (2, 256, 34816) and (16, 256, 17408): the small-M kernel with K split
# eight ways, fused quantization and a separate cast
@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (3, 1024, 1024), (16, 1024, 1024), (8, 4096, 4096),
                                   (2, 256, 34816), (16, 256, 17408),
                                   (1024, 4096, 4096), (130, 272, 400), (300, 2048, 4096),
                                   (520, 4208, 8000)])
def test_fp8_linear_graph(M, N, K, fast):
    g = wl.rng(11, M, N)
    pw = bql.prepack_weight(dev16(wl.weight(g, N, K, "bf16"), "bf16"), "fp8_tensor")
    a = dev16(wl.activation(g, M, K, "bf16", "channels"), "bf16")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(256, bql.fp8_linear_workspace_size(M, N, K)), dtype=torch.uint8, device=DEV)
    scale = torch.empty(1, dtype=torch.float32, device=DEV)
    other = torch.empty_like(out)

    def run():
        bql.fp8_linear(a, pw, a_scale=scale, out_dtype=torch.bfloat16, out=out, ws=ws, fast_accum=fast)

    def noise():  # eager work on the same library between replays
        bql.fp8_linear(a * 2, pw, out_dtype=torch.bfloat16, out=other, fast_accum=fast)

    _replays_match(run, out, noise)


def test_w8a16_and_w4a8_graph():
    g = wl.rng(12, 0)
    N = K = 1024
    pw16 = bql.prepack_weight(dev16(wl.weight(g, N, K, "f16"), "f16"), "fp8_channel")
    a16 = dev16(wl.activation(g, 8, K, "f16"), "f16")
    out16 = torch.empty((8, N), dtype=torch.float16, device=DEV)
    _replays_match(lambda: bql.w8a16_linear(a16, pw16, out=out16), out16,
                   lambda: bql.w8a16_linear(a16 * 3, pw16))
    w4 = wl.int4_weight(g, N, K)
    pw4 = bql.prepack_weight(dev(wl.pack_int4(w4).reshape(N, K // 2)), "int4_channel",
                             scales=dev16(wl.w4a8_channel_scales(g, N), "f16"))
    aq = dev(g.integers(-127, 128, (200, K), dtype=np.int8))
    out4 = torch.empty((200, N), dtype=torch.int32, device=DEV)
    ws4 = torch.empty(max(256, bql.lib().bql_w4a8_linear_workspace_size(200, N, K)), dtype=torch.uint8,
                      device=DEV)
    _replays_match(lambda: bql.w4a8_linear(aq, None, pw4, out_dtype=torch.int32, out=out4, ws=ws4), out4,
                   lambda: bql.w4a8_linear(aq, None, pw4, out_dtype=torch.int32))


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (16, 1024, 1024), (512, 1024, 4096)])
def test_fp8_linear_static_graph(M, N, K):
    g = wl.rng(13, M, N)
    pw = bql.prepack_weight(dev16(wl.weight(g, N, K, "bf16"), "bf16"), "fp8_channel")
    a = dev16(wl.activation(g, M, K, "bf16", "channels"), "bf16")
    sa = torch.tensor([0.01], dtype=torch.float32, device=DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(256, bql.fp8_linear_workspace_size(M, N, K)), dtype=torch.uint8, device=DEV)
    _replays_match(lambda: bql.fp8_linear_static(a, pw, sa, out_dtype=torch.bfloat16, out=out, ws=ws),
                   out, lambda: bql.fp8_linear_static(a * 2, pw, sa, out_dtype=torch.bfloat16))


@pytest.mark.parametrize("M", [1, 300])
def test_small_n_graph(M):
    N, K = 8, 4096
    g = wl.rng(14, M)
    pw = bql.prepack_weight(dev16(wl.weight(g, N, K, "bf16"), "bf16"), "fp8_tensor")
    a = dev16(wl.activation(g, M, K, "bf16", "channels"), "bf16")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(256, bql.fp8_linear_workspace_size(M, N, K)), dtype=torch.uint8, device=DEV)
    _replays_match(lambda: bql.fp8_linear(a, pw, out_dtype=torch.bfloat16, out=out, ws=ws), out,
                   lambda: bql.fp8_linear(a * 3, pw, out_dtype=torch.bfloat16))


def test_rmsnorm_quantizers_graph():
    M, K = 256, 4096
    g = wl.rng(15, 0)
    x = dev16(wl.activation(g, M, K, "bf16", "channels"), "bf16")
    gw = dev16(wl.norm_weight(g, K, "bf16"), "bf16")
    q8 = torch.empty((M, K), dtype=torch.int8, device=DEV)
    s8 = torch.empty(M, dtype=torch.float32, device=DEV)
    L = bql.lib()

    def run8():
        bql._check("int8", L.bql_rmsnorm_int8_quantize_per_token(
            bql._ptr(x), bql._ptr(gw), bql.BF16, M, K, 1e-5, bql._ptr(q8), bql._ptr(s8), None,
            bql._stream(x.device)))
    _replays_match(run8, q8, lambda: bql.rmsnorm_int8_quantize_per_token(x * 2, gw, 1e-5))
    qf = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    sf = torch.empty(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(256, L.bql_rmsnorm_quantize_workspace_size(M)), dtype=torch.uint8, device=DEV)

    def runf():
        bql._check("fp8", L.bql_rmsnorm_fp8_quantize_dynamic(
            bql._ptr(x), bql._ptr(gw), bql.BF16, M, K, 1e-5, bql._ptr(qf), bql._ptr(sf), None,
            bql._ptr(ws), ws.numel(), bql._stream(x.device)))
    _replays_match(runf, qf, lambda: bql.rmsnorm_fp8_quantize_dynamic(x * 3, gw, 1e-5))


@pytest.mark.parametrize("M", [1, 200])
def test_w4a8_group_graph(M):
    N, K = 1024, 1024
    g = wl.rng(16, M)
    w4 = wl.int4_weight(g, N, K)
    sc = dev((g.uniform(0.5, 2.0, size=(N, K // 128)) * 2.0 ** -8).astype(np.float32))
    pw = bql.prepack_weight(dev(wl.pack_int4(w4).reshape(N, K // 2)), "int4_group", scales=sc)
    aq = dev(g.integers(-127, 128, (M, K), dtype=np.int8))
    sa = dev(g.uniform(1e-3, 1e-1, size=M).astype(np.float32))
    out = torch.empty((M, N), dtype=torch.float16, device=DEV)
    ws = torch.empty(max(256, bql.lib().bql_w4a8_linear_workspace_size(M, N, K)), dtype=torch.uint8,
                     device=DEV)
    _replays_match(lambda: bql.w4a8_group_linear(aq, sa, pw, out=out, ws=ws), out,
                   lambda: bql.w4a8_group_linear(aq, sa * 2, pw))


@pytest.mark.parametrize("M,N,K", [(100, 1024, 1040), (64, 272, 400)])
def test_prequantized_ksplit_graph(M, N, K):
    # E4M3 A at 16 < M <= 128 with few output tiles: the k-split kernel
    # gathers A row-major where it is (no repack launch); ragged K
    g = np.random.Generator(np.random.PCG64(M + K))
    codes = g.integers(0, 256, (M, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    pw = bql.prepack_weight(dev16(wl.weight(wl.rng(17, N), N, K, "bf16"), "bf16"), "fp8_channel")
    a = dev(codes).view(torch.float8_e4m3fn)
    sa = torch.tensor([0.02], dtype=torch.float32, device=DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(256, bql.fp8_linear_workspace_size(M, N, K)), dtype=torch.uint8, device=DEV)
    other = torch.empty_like(out)
    _replays_match(lambda: bql.fp8_linear(a, pw, a_scale=sa, out_dtype=torch.bfloat16, out=out, ws=ws),
                   out, lambda: bql.fp8_linear(a, pw, a_scale=sa * 2, out_dtype=torch.bfloat16, out=other))


def test_packed_activations_graph():
    # pre-packed E4M3 A (BQL_E4M3_TILES) into the exact tile kernel, K split
    M, N, K = 520, 4208, 8000
    g = np.random.Generator(np.random.PCG64(M + N + K))
    codes = g.integers(0, 256, (M, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    pw = bql.prepack_weight(dev16(wl.weight(wl.rng(19, N), N, K, "bf16"), "bf16"), "fp8_tensor")
    pa = bql.pack_activations(dev(codes))
    sa = torch.tensor([0.02], dtype=torch.float32, device=DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(256, bql.fp8_linear_workspace_size(M, N, K)), dtype=torch.uint8, device=DEV)
    other = torch.empty_like(out)
    _replays_match(lambda: bql.fp8_linear(pa, pw, a_scale=sa, out_dtype=torch.bfloat16, out=out, ws=ws),
                   out, lambda: bql.fp8_linear(pa, pw, a_scale=sa * 2, out_dtype=torch.bfloat16, out=other))

