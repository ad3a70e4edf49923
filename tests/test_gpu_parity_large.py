"""Bit-exact parity at the workloads' full sizes for the codes the linears
consume: the prepacked weight codes of the large Llama shapes, and the
activation codes the dynamic per-tensor quantizer writes inside
bql_fp8_linear.

The weight is quantized after load with a per-tensor scale (vLLM PR #4118,
"Algorithm") or a scale per output channel (optimum-quanto PR #241), and the
activation is quantized every call with scale = amax / 448 and a saturating
round-to-nearest-even E4M3 cast (vLLM PR #4118, "Algorithm").  Codes and
scales must equal the oracle's bit for bit, at every element.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import DEV, dev16, host, say

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu


# the Llama-3-8B up-projection (per tensor) and the Llama-70B prefill shapes
# (per channel), as the fp8 linear workloads use them
@pytest.mark.parametrize("N,K,fmt,cfg,idx", [
    (28672, 4096, "fp8_tensor", 3, 2),
    (10240, 8192, "fp8_channel", 4, 0),
    (57344, 8192, "fp8_channel", 4, 2),
    (8192, 28672, "fp8_channel", 4, 3),
])
def test_prepacked_codes_full_size(N, K, fmt, cfg, idx):
    say(f"prepack {fmt} N={N} K={K}")
    bits = wl.weight(wl.rng(cfg, idx, 1), N, K, "bf16")
    pw = bql.prepack_weight(dev16(bits, "bf16"), fmt)
    codes = host(bql.unpack_weight(pw))
    del pw
    torch.cuda.empty_cache()
    wf = oracle.decode_input(bits, "bf16")
    del bits
    if fmt == "fp8_tensor":
        q, s = oracle.quant_per_tensor(wf)
    else:
        q, s = oracle.quant_per_row(wf)
    del wf
    assert np.array_equal(codes, q), f"{int((codes != q).sum())} codes differ"


def _unpack_activation_tiles(buf: np.ndarray, M: int, K: int) -> np.ndarray:
    """Logical [M, K] codes from the packed activation layout the dynamic
    quantizer writes into the fp8 linear's workspace (after its 8 KiB of
    amax partials and scale): 16-row x 128-k tiles of 2 KiB, all k-tiles of
    a 16-row strip in a row; inside a tile [half h][lane l][16 bytes], lane
    l holding row l % 16 and k = 32 (l // 16) + 16 h + j."""
    mt, kt = (M + 15) // 16, (K + 127) // 128
    t = buf[: mt * kt * 2048].reshape(mt, kt, 2, 4, 16, 16)  # strip, ktile, h, lane//16, lane%16, j
    # -> strip, lane%16 (row), ktile, lane//16, h, j  (k = 128 kt + 32 g + 16 h + j)
    logical = t.transpose(0, 4, 1, 3, 2, 5).reshape(mt * 16, kt * 128)
    return logical[:M, :K]


def _check_in_linear_codes(a_bits, dtype, M, N, K, wbits, nan_sign_free=False):
    """The scale and the packed codes of a bql_fp8_linear call's in-linear
    quantizer equal the oracle's; with nan_sign_free, a NaN code may carry
    either sign (the sign of a NaN made by a division is not fixed by IEEE
    754), every other code must be identical."""
    pw = bql.prepack_weight(dev16(wbits, "bf16"), "fp8_tensor")
    ws = torch.zeros(bql.fp8_linear_workspace_size(M, N, K), dtype=torch.uint8, device=DEV)
    sa = torch.empty(1, dtype=torch.float32, device=DEV)
    bql.fp8_linear(dev16(a_bits, dtype), pw, a_scale=sa, ws=ws)
    torch.cuda.synchronize()
    wsb = host(ws)
    scale_in_ws = wsb[4096:4100].view(np.float32)[0]
    got = _unpack_activation_tiles(wsb[8192:], M, K)
    with np.errstate(invalid="ignore"):
        aq, sa_ref = oracle.quant_per_tensor(oracle.decode_input(a_bits, dtype))
    same_scale = (lambda x, y: x.view(np.uint32) == y.view(np.uint32) or (np.isnan(x) and np.isnan(y)))
    assert same_scale(host(sa)[0], np.float32(sa_ref))
    assert same_scale(np.float32(scale_in_ws), np.float32(sa_ref))
    if nan_sign_free:
        nan = (aq & 0x7F) == 0x7F
        assert np.array_equal((got & 0x7F) == 0x7F, nan), "NaN codes differ"
        got, aq = got[~nan], aq[~nan]
    assert np.array_equal(got, aq), f"{int((got != aq).sum())} codes differ"
    return aq


@pytest.mark.parametrize("M,N,K", [(1024, 4096, 14336), (4096, 8192, 28672)])
def test_in_linear_activation_codes(M, N, K):
    # the quantizer's codes as the tile kernels read them, read back from
    # the workspace of a bql_fp8_linear call with bf16 activations
    say(f"in-linear activation codes M={M} N={N} K={K}")
    cfg, idx = (3, 3) if K == 14336 else (4, 3)
    a_bits = wl.activation(wl.rng(cfg, idx, M, 3), M, K, "bf16", "channels")
    wbits = wl.weight(wl.rng(cfg, idx, 1), N, K, "bf16")
    aq = _check_in_linear_codes(a_bits, "bf16", M, N, K, wbits)
    say(f"  {M * K} codes identical, saturated {np.mean((aq & 0x7F) == 0x7E):.2e}")


# Small activations: the small-M kernel's packed input (16, 4096) and
# (24, 2048) in fp16, the tile kernels' at a ragged row strip and k-tile
# (40, 6544) and (65, 4096).
@pytest.mark.parametrize("M,N,K,dtype", [(16, 1024, 4096, "bf16"), (24, 1040, 2048, "f16"),
                                         (40, 1040, 6544, "bf16"), (65, 1024, 4096, "bf16")])
def test_in_linear_activation_codes_small(M, N, K, dtype):
    g = wl.rng(97, M, K)
    a_bits = wl.activation(g, M, K, dtype, "channels")
    _check_in_linear_codes(a_bits, dtype, M, N, K, wl.weight(g, N, K, "bf16"))


@pytest.mark.parametrize("M,K", [(16, 2048), (80, 4096)])
@pytest.mark.parametrize("kind", ["zeros", "inf", "nan"])
def test_in_linear_activation_codes_special(kind, M, K):
    # a zero tensor (scale 1, zero codes), an infinity (infinite scale: codes
    # of x / inf, NaN for the infinity itself) and a NaN (NaN scale: NaN
    # codes) through the in-linear quantizer of the small-M kernel (16 x
    # 2048) and of the tile kernels (80 x 4096)
    N = 1024
    g = wl.rng(98, M, K)
    a = oracle.decode_input(wl.activation(g, M, K, "bf16", "channels"), "bf16").astype(np.float32)
    if kind == "zeros":
        a[:] = 0.0
    else:
        a[5, 777] = np.inf if kind == "inf" else np.nan
    _check_in_linear_codes(wl.to_bits(a, "bf16"), "bf16", M, N, K, wl.weight(g, N, K, "bf16"),
                           nan_sign_free=True)


def test_unpack_helper_layout():
    # the host-side unpack of the test against a layout built by hand: tile
    # (strip 1, k-tile 0), half 1, lane 20, byte 3 holds row 16 + 4,
    # k = 32 * 1 + 16 + 3 = 51
    M, K = 32, 256
    buf = np.zeros(2 * 2 * 2048, dtype=np.uint8)
    strip, kt, h, lane, j = 1, 0, 1, 20, 3
    buf[(strip * 2 + kt) * 2048 + h * 1024 + lane * 16 + j] = 77
    out = _unpack_activation_tiles(buf, M, K)
    assert out[20, 51] == 77 and int(out.sum()) == 77
