"""GPU parity at the largest reductions the linears accept, against the CPU
oracle.

fp8 linear at K = 2^22 (the bql_fp8_linear limit), N = 16: the small-M
path with fused dynamic quantization (M = 1), the tile path with dynamic
quantization and with pre-quantized E4M3 A (M = 40).  W4A8 at K = 131056
(the limit that keeps 16 * acc inside int32 for every int8 code, -128
included), int32 accumulators compared bit for bit, with every product of
the first row and channel at the largest magnitude, -128 * -8, so that the
sum reaches its extreme.  Per-group W4A8 at K = 16384 (128 groups,
the limit of the staged scales).  W8A16 at K = 2^24, the limit of the
weight formats.  Both RMSNorm quantizers at M = 2^22, the row limit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import DEV, assert_close, dev, dev16, host, host_f64, say

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu

K_FP8 = 1 << 22
K_W4A8 = 131056
K_GROUP = 16384


@pytest.fixture(scope="module")
def fp8_case():
    g = wl.rng(120, 0)
    N = 16
    wb = wl.weight(g, N, K_FP8, "bf16")
    ab = wl.activation(g, 40, K_FP8, "bf16", "channels")
    wq, sw = oracle.quant_per_tensor(oracle.decode_input(wb, "bf16"))
    pw = bql.prepack_weight(dev16(wb, "bf16"), "fp8_tensor")
    return wb, ab, wq, sw, pw


@pytest.mark.parametrize("M", [1, 40])
def test_fp8_linear_max_k_dynamic(fp8_case, M):
    _, ab, wq, sw, pw = fp8_case
    sa = torch.empty(1, dtype=torch.float32, device=DEV)
    y = bql.fp8_linear(dev16(ab[:M], "bf16"), pw, a_scale=sa, out_dtype=torch.float32)
    torch.cuda.synchronize()
    aq, sa_ref = oracle.quant_per_tensor(oracle.decode_input(ab[:M], "bf16"))
    assert sa.item() == float(sa_ref), "activation scale differs"
    assert_close(host_f64(y), oracle.fp8_linear(aq, sa_ref, wq, sw), f"fp8 K=2^22 M={M}")
    say(f"  fp8 linear M={M} N=16 K=2^22 within tolerance")


def test_fp8_linear_max_k_prequantized(fp8_case):
    _, ab, wq, sw, pw = fp8_case
    aq, sa = oracle.quant_per_tensor(oracle.decode_input(ab, "bf16"))
    y = bql.fp8_linear(dev(aq).view(torch.float8_e4m3fn), pw, a_scale=torch.tensor([sa], device=DEV),
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(host_f64(y), oracle.fp8_linear(aq, sa, wq, sw), "fp8 K=2^22 M=40 E4M3 A")


@pytest.mark.parametrize("M", [1, 40])
def test_w4a8_max_k_extreme_sum(M):
    # row 0 of A and channel 0 of W hold -128 and -8 throughout: acc[0, 0] =
    # 1024 * K, i.e. 16 * acc = 2^31 - 2^18, the top of the int32 range the
    # int8 MMA works in; sign changes elsewhere make the other entries differ
    N = 16
    w4 = np.full((N, K_W4A8), -8, dtype=np.int8)
    aq = np.full((M, K_W4A8), -128, dtype=np.int8)
    aq[1:, ::7] = 127
    w4[1::2, ::5] = 7
    pw = bql.prepack_weight(torch.from_numpy(wl.pack_int4(w4).reshape(N, K_W4A8 // 2)).to(DEV),
                            "int4_channel", scales=torch.ones(N, dtype=torch.float16, device=DEV))
    acc = bql.w4a8_linear(dev(aq), None, pw, out_dtype=torch.int32)
    torch.cuda.synchronize()
    ref = oracle.w4a8_acc(aq, w4)
    assert ref[0, 0] * 16 == 2 ** 31 - 2 ** 18, "the case must reach the documented extreme"
    assert np.array_equal(host(acc).astype(np.int64), ref), f"W4A8 K={K_W4A8} M={M} accumulators differ"


@pytest.mark.parametrize("M", [1, 40])
def test_w4a8_group_max_k(M):
    N = 32
    g = wl.rng(121, M)
    w4 = wl.int4_weight(g, N, K_GROUP)
    sw = (g.uniform(0.5, 2.0, size=(N, K_GROUP // 128)) * 2.0 ** -8).astype(np.float32)
    pw = bql.prepack_weight(torch.from_numpy(wl.pack_int4(w4).reshape(N, K_GROUP // 2)).to(DEV),
                            "int4_group", scales=dev(sw))
    aq = g.integers(-127, 128, size=(M, K_GROUP), dtype=np.int8)
    sa = g.uniform(1e-3, 1e-1, size=M).astype(np.float32)
    y = bql.w4a8_group_linear(dev(aq), dev(sa), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(host_f64(y), oracle.w4a8_group_linear(aq, sa, w4, sw), f"g128 K={K_GROUP} M={M}")


@pytest.mark.parametrize("M", [1, 8])
def test_w8a16_max_k(M):
    # K = 2^24, the limit of the weight formats; per-channel fp16 scales
    N, K = 16, 1 << 24
    g = wl.rng(122, M)
    wb = wl.weight(g, N, K, "f16")
    wf = oracle.decode_input(wb, "f16")
    sbits = wl.w8a16_channel_scales(g, wf)
    s32 = oracle.decode_input(sbits, "f16")
    pw = bql.prepack_weight(dev16(wb, "f16"), "fp8_channel", scales=dev16(sbits, "f16"))
    ab = wl.activation(g, M, K, "f16")
    y = bql.w8a16_linear(dev16(ab, "f16"), pw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.w8a16_linear(oracle.decode_input(ab, "f16"), oracle.quant_with_scales(wf, s32), s32)
    assert_close(host_f64(y), ref, f"W8A16 K=2^24 M={M}")


def test_rmsnorm_quantizers_max_m():
    # M = 2^22 (the row limit) with K = 32: every block of the persistent
    # grid walks about 4096 rows, and the E4M3 cast folds 1024 block maxima
    M, K = 1 << 22, 32
    g = wl.rng(123, 0)
    xb = wl.activation(g, M, K, "f16", "entries")
    gb = wl.norm_weight(g, K, "f16")
    x = oracle.decode_input(xb, "f16")
    gf = oracle.decode_input(gb, "f16")
    lo, hi = oracle.rms_inv_candidates(x, 1e-5)
    q8, s8, r8 = bql.rmsnorm_int8_quantize_per_token(dev16(xb, "f16"), dev16(gb, "f16"), 1e-5, inv_rms=True)
    qf, sf, rf = bql.rmsnorm_fp8_quantize_dynamic(dev16(xb, "f16"), dev16(gb, "f16"), 1e-5, inv_rms=True)
    torch.cuda.synchronize()
    for r in (host(r8), host(rf)):
        assert ((r == lo) | (r == hi)).all(), "inadmissible 1/rms"
    q_ref, s_ref, _ = oracle.rmsnorm_int8_per_token(x, gf, 1e-5, r=host(r8))
    assert np.array_equal(host(s8).view(np.uint32), s_ref.view(np.uint32)), "int8 scales differ"
    assert np.array_equal(host(q8), q_ref), "int8 codes differ"
    qf_ref, sf_ref, _ = oracle.rmsnorm_fp8_per_tensor(x, gf, 1e-5, r=host(rf))
    assert host(sf).view(np.uint32)[0] == np.float32(sf_ref).view(np.uint32), "E4M3 scale differs"
    assert np.array_equal(host(qf), qf_ref), "E4M3 codes differ"
