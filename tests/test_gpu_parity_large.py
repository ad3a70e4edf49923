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


@pytest.mark.parametrize("M,N,K", [(1024, 4096, 14336), (4096, 8192, 28672)])
def test_in_linear_activation_codes(M, N, K):
    # the quantizer's codes as the tile kernels read them, read back from
    # the workspace of a bql_fp8_linear call with bf16 activations
    say(f"in-linear activation codes M={M} N={N} K={K}")
    cfg, idx = (3, 3) if K == 14336 else (4, 3)
    a_bits = wl.activation(wl.rng(cfg, idx, M, 3), M, K, "bf16", "channels")
    wbits = wl.weight(wl.rng(cfg, idx, 1), N, K, "bf16")
    pw = bql.prepack_weight(dev16(wbits, "bf16"), "fp8_tensor")
    ws = torch.zeros(bql.fp8_linear_workspace_size(M, N, K), dtype=torch.uint8, device=DEV)
    sa = torch.empty(1, dtype=torch.float32, device=DEV)
    bql.fp8_linear(dev16(a_bits, "bf16"), pw, a_scale=sa, ws=ws)
    torch.cuda.synchronize()
    wsb = host(ws)
    scale_in_ws = wsb[4096:4100].view(np.float32)[0]
    got = _unpack_activation_tiles(wsb[8192:], M, K)
    aq, sa_ref = oracle.quant_per_tensor(oracle.decode_input(a_bits, "bf16"))
    assert host(sa)[0].view(np.uint32) == np.float32(sa_ref).view(np.uint32)
    assert np.float32(scale_in_ws).view(np.uint32) == np.float32(sa_ref).view(np.uint32)
    assert np.array_equal(got, aq), f"{int((got != aq).sum())} codes differ"
    say(f"  {M * K} codes identical, saturated {np.mean((aq & 0x7F) == 0x7E):.2e}")


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
