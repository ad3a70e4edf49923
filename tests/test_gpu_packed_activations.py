"""GPU parity of pre-packed E4M3 activations: bql_fp8_pack_activations and
bql_fp8_linear with adt = BQL_E4M3_TILES.

Pre-quantized activation codes (vLLM PR #4118, "Algorithm": per-tensor
scale amax / 448, saturating nearest-even E4M3) are packed once into the
operand-tile layout; the linear then reads them as they are.  The packed
buffer must hold exactly the codes (unpacked on the host, every element,
zeros past M and K), and the linear on packed A must equal the linear on the
same row-major codes bit for bit (same kernels, same sums) and the oracle
within |d| <= 5e-3 (|ref| + 1e-2 max|ref|): for the exact tile kernel at
several block widths and K splits, the k-split kernel (M <= 128) and the fast
fp8 kernels.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _common import DEV, Weights, assert_close, dev, dev16, host, host_f64, rows_for, say

import bit_quantized_linear_amd as bql

pytestmark = pytest.mark.gpu


def _logical(buf: np.ndarray, M: int, K: int) -> np.ndarray:
    """[Mpad, Kpad] codes of the tile layout: 16-row x 128-k tiles of 2 KiB,
    a strip's k-tiles in a row; in a tile, half h, lane l = r + 16 g holds
    row r, k = 32 g + 16 h .. +15."""
    mt, kt = (M + 15) // 16, (K + 127) // 128
    t = buf[: mt * kt * 2048].reshape(mt, kt, 2, 4, 16, 16)
    return t.transpose(0, 4, 1, 3, 2, 5).reshape(mt * 16, kt * 128)


@pytest.mark.parametrize("M,K", [(17, 128), (300, 4000), (1024, 14336)])
def test_pack_layout_holds_the_codes(M, K):
    g = np.random.Generator(np.random.PCG64(M * 7 + K))
    codes = g.integers(0, 256, size=(M, K), dtype=np.uint8)
    pa = bql.pack_activations(dev(codes))
    torch.cuda.synchronize()
    got = _logical(host(pa.packed), M, K)
    assert np.array_equal(got[:M, :K], codes)
    assert not got[M:, :].any() and not got[:, K:].any(), "padding must hold zero codes"


@pytest.mark.parametrize("M,N,K,fast", [
    (1024, 6144, 4096, False),    # exact tile kernel, 256 x 96 blocks
    (1024, 4096, 14336, False),   # exact tile kernel, K split four ways
    (777, 2096, 4000, False),     # exact, ragged M and K, K split
    (128, 2048, 4096, False),     # k-split exact kernel (M <= 128)
    (1024, 28672, 4096, True),    # fast fp8 256 x 256 kernel
    (200, 1040, 8192, True),      # fast fp8 register-prefetch kernel, K split
])
def test_linear_on_packed_activations(M, N, K, fast):
    say(f"packed A: M={M} N={N} K={K} fast={fast}")
    W = Weights(141, N + K + M, N, K, "bf16", M % 2 == 0)
    pw = bql.prepack_weight(dev16(W.bits, "bf16"), "fp8_channel" if W.scales.size > 1 else "fp8_tensor")
    a_bits = wl.activation(wl.rng(141, M, N, K), M, K, "bf16", "channels")
    q, sa = bql.quantize_dynamic(dev16(a_bits, "bf16"))
    q = q.view(torch.float8_e4m3fn)
    pa = bql.pack_activations(q)
    y_row = bql.fp8_linear(q, pw, a_scale=sa, out_dtype=torch.float32, fast_accum=fast)
    y_pk = bql.fp8_linear(pa, pw, a_scale=sa, out_dtype=torch.float32, fast_accum=fast)
    torch.cuda.synchronize()
    assert torch.equal(y_row.view(torch.int32), y_pk.view(torch.int32)), "packed and row-major A differ"
    if not fast:
        aq_ref, sa_ref = oracle.quant_per_tensor(oracle.decode_input(a_bits, "bf16"))
        rows = rows_for(M, 500 + M, 16)
        y_ref = oracle.fp8_linear(aq_ref, sa_ref, W.codes, W.scales, rows=rows)
        assert_close(host_f64(y_pk)[rows], y_ref, f"packed A M={M} N={N} K={K}")


def test_small_m_rejects_packed_activations():
    pa = bql.pack_activations(torch.zeros((16, 256), dtype=torch.uint8, device=DEV))
    pw = bql.prepack_weight(torch.zeros((64, 256), dtype=torch.bfloat16, device=DEV), "fp8_tensor")
    with pytest.raises(bql.BQLError, match="BQL_ERR_SHAPE"):
        bql.fp8_linear(pa, pw, a_scale=torch.ones(1, device=DEV))
