"""GPU parity of the exact fp8 tile kernel for M > 128 (blocks of 256 rows
by 32 fn columns, each wave 128 rows by fn 16-column strips, K split over
blocks where the planner says so), against the CPU oracle.

The fp8 linear Y = (sA sW[n]) (Aq Wq^T) of vLLM PR #4118 with dynamic
per-tensor activation scaling, exact products summed in fp32.  Covered:
every block width the planner uses (fn = 2, 3, 4, 6, 7, 8) with 1 to 4 K
splits, the Llama-3-8B projections at M = 1024, ragged M / N / K (partial
row and column tiles, K padded inside the operand tiles), fp32 and fp8
outputs (vLLM discussion #5802, output_scale), per-channel weight scales
(optimum-quanto PR #241) and pre-quantized E4M3 activations.  Float
outputs within |d| <= 5e-3 (|ref| + 1e-2 max|ref|) on seeded sampled rows;
activation scales identical.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import (DEV, Weights, assert_close, assert_fp8_out, dev16, exact_plan, host, host_f64,
                     rows_for, say)

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu


def _run(M, N, K, idx, per_channel=False, out_dtype=torch.bfloat16, prequant=False, fp8_out=False):
    say(f"exact tile: M={M} N={N} K={K} plan={exact_plan(M, N, K)} per_channel={per_channel} "
        f"out={out_dtype} prequant={prequant} fp8_out={fp8_out}")
    assert exact_plan(M, N, K)[0] != 0, "shape must select the exact tile kernel"
    W = Weights(97, idx, N, K, "bf16", per_channel)
    pw = bql.prepack_weight(dev16(W.bits, "bf16"), "fp8_channel" if per_channel else "fp8_tensor")
    assert np.array_equal(host(pw.scales).view(np.uint32), W.scales.view(np.uint32))
    a_bits = wl.activation(wl.rng(97, idx, M, 3), M, K, "bf16", "channels")
    a = dev16(a_bits, "bf16")
    aq_ref, sa_ref = oracle.quant_per_tensor(oracle.decode_input(a_bits, "bf16"))
    rows = rows_for(M, 700 + M, 24)
    y_ref = oracle.fp8_linear(aq_ref, sa_ref, W.codes, W.scales, rows=rows)
    if prequant:
        q, sa = bql.quantize_dynamic(a)
        y = bql.fp8_linear(q.view(torch.float8_e4m3fn), pw, a_scale=sa, out_dtype=out_dtype)
    else:
        sa = torch.empty(1, dtype=torch.float32, device=DEV)
        y = bql.fp8_linear(a, pw, a_scale=sa, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert host(sa)[0].view(np.uint32) == np.float32(sa_ref).view(np.uint32)
    assert_close(host_f64(y)[rows], y_ref, f"M={M} N={N} K={K}")
    if fp8_out:
        for mult in (1.0, 0.5):  # 0.5: part of the output saturates
            osc = np.float32(np.abs(y_ref).max() / 448.0 * mult)
            yq = bql.fp8_linear(a, pw, out_dtype=torch.float8_e4m3fn,
                                output_scale=torch.tensor([osc], device=DEV))
            torch.cuda.synchronize()
            assert_fp8_out(host(yq)[rows], y_ref / np.float64(osc), f"  fp8 out x{mult}")


def test_llama3_up_projection_m1024():
    _run(1024, 28672, 4096, 0)


def test_ragged_rows_columns_and_k():
    # 777 rows: a partial 256-row tile and a partial 16-row strip; N = 30032:
    # a partial 256-column tile; K = 4000: k-tiles padded with zero codes
    _run(777, 30032, 4000, 1)


def test_fp32_and_fp8_outputs():
    _run(600, 32768, 1024, 2, out_dtype=torch.float32, fp8_out=True)


def test_per_channel_weight_scales():
    _run(1024, 24576, 2048, 3, per_channel=True)


def test_prequantized_e4m3_activations():
    _run(1024, 28672, 4096, 4, prequant=True)


# (M, N, K) -> (fn, splits): each block width and split count the planner
# uses, with partial row tiles (M % 256 != 0), partial column blocks and K
# not a multiple of 128
PLANS = [((520, 1040, 1008), (2, 1)), ((520, 1040, 2000), (2, 4)), ((520, 5792, 1008), (3, 1)),
         ((520, 2192, 3008), (3, 3)), ((520, 8432, 1008), (4, 1)), ((777, 2096, 4000), (4, 3)),
         ((520, 11072, 1008), (6, 1)), ((520, 7376, 8000), (6, 2)), ((520, 16352, 1008), (7, 1)),
         ((520, 4208, 8000), (7, 4)), ((520, 19520, 1008), (8, 1)), ((520, 9488, 14336), (8, 2))]


@pytest.mark.parametrize("shape,plan", PLANS)
def test_every_block_width_and_split(shape, plan):
    # split shapes also check the fp8 output (the reduce's epilogue); every
    # other shape takes per-channel weight scales
    i = PLANS.index((shape, plan))
    assert exact_plan(*shape) == plan
    _run(*shape, 10 + i, per_channel=i % 2 == 1, fp8_out=plan[1] > 1)


# the Llama-3-8B projections of the fp8 step at M = 1024
@pytest.mark.parametrize("N,K", [(6144, 4096), (4096, 4096), (4096, 14336)])
def test_llama3_projections_m1024(N, K):
    _run(1024, N, K, 30 + N + K)


def test_single_k_tile():
    # K = 128: two half-steps only (the shortest pipeline)
    _run(520, 49152, 128, 5)


@pytest.mark.parametrize("M,N,K", [(640, 49152, 512), (777, 2096, 4000)])
def test_deterministic(M, N, K):
    W = Weights(97, 6, N, K, "bf16", False)
    pw = bql.prepack_weight(dev16(W.bits, "bf16"), "fp8_tensor")
    a = dev16(wl.activation(wl.rng(97, 6, M, 3), M, K, "bf16", "channels"), "bf16")
    y0 = bql.fp8_linear(a, pw)
    y1 = bql.fp8_linear(a, pw)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
