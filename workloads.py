"""Seeded synthetic inputs shared by the tests, the smoke check and bench.py.

This module holds only random-number generation and storage formatting
(fp32 -> fp16/bf16 bit patterns, int4 nibble packing).  It contains none of
the quantization or linear-algebra arithmetic of the method: no scale
formula, no E4M3 rounding, no dot product.  Both the CPU oracle and the HIP
path receive the same arrays from here.

Workloads (shapes follow the pages' linear layers; values are synthetic, no
checkpoint or dataset is involved):
  cfg1  W8A8 fp8 linear, M=16, K=N=1024: A fp16 ~N(0,1) with 1% of entries
        multiplied by 20; W fp16 ~N(0, 0.02) quantized per tensor.
  cfg2  W8A16 decode GEMV, M in {1, 8}, K=N=4096: A fp16 ~N(0,1); W fp16
        ~N(0, 0.02); per-channel fp16 scales u_n * max|W[n,:]| / 448 with
        u_n ~ U[0.5, 2].
  cfg3  Llama-3-8B-shaped W8A8 linears, bf16, (N,K) in {(6144,4096),
        (4096,4096), (28672,4096), (4096,14336)}, M in {1,16,128,1024}; A
        ~N(0,1) with 1% of the K columns multiplied by 20; W ~N(0, 0.02).
  cfg4  Llama-70B-shaped W8A8 prefill, bf16, (N,K) in {(10240,8192),
        (8192,8192), (57344,8192), (8192,28672)}, M in {1024, 4096},
        per-channel weight scales.
  cfg5  W4A8, K=N in {4096,5120,6656,8192}, M in {1,16,256,1024}: W int4
        ~U{-8..7}; A fp16 ~N(0,1) (quantized per token by each side); weight
        scales fp16 ~U[0.5,2] * 2^-8.
  RMSNorm ahead of the quantizers: the activation recipe above as the
        norm's input, gain g ~U[0.5, 1.5] in the activation dtype.
"""
from __future__ import annotations

import numpy as np

CFG3_SHAPES = [(6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336)]
CFG3_M = [1, 16, 128, 1024]
CFG4_SHAPES = [(10240, 8192), (8192, 8192), (57344, 8192), (8192, 28672)]
CFG4_M = [1024, 4096]
CFG5_KN = [4096, 5120, 6656, 8192]
CFG5_M = [1, 16, 256, 1024]


def rng(cfg: int, *fold: int) -> np.random.Generator:
    """PCG64 stream for config `cfg` (seed 1000 + cfg) with shape indices folded in."""
    return np.random.Generator(np.random.PCG64([1000 + cfg, *[int(f) for f in fold]]))


# ------------------------------------------------------- storage formats

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even) and return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return f32_to_f16_bits(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def pack_int4(w: np.ndarray) -> np.ndarray:
    """Logical int4 packing: two's-complement nibbles, low nibble = even k."""
    w = np.asarray(w, dtype=np.int8)
    N, K = w.shape
    assert K % 2 == 0
    nib = (w.astype(np.int16) & 15).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).reshape(N * K // 2)


# ------------------------------------------------------------ generators

def activation(g: np.random.Generator, M: int, K: int, dtype: str,
               outliers: str = "none", factor: float = 20.0, frac: float = 0.01) -> np.ndarray:
    """A ~ N(0,1) as fp16/bf16 bits [M,K]; optional outlier entries or K-columns."""
    a = g.standard_normal((M, K), dtype=np.float32)
    if outliers == "entries":
        a = np.where(g.random((M, K)) < frac, a * factor, a).astype(np.float32)
    elif outliers == "channels":
        cols = g.random(K) < frac
        a[:, cols] *= factor
    elif outliers != "none":
        raise ValueError(outliers)
    return to_bits(a, dtype)


def weight(g: np.random.Generator, N: int, K: int, dtype: str, std: float = 0.02) -> np.ndarray:
    w = g.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    return to_bits(w, dtype)


def w8a16_channel_scales(g: np.random.Generator, w_f32: np.ndarray) -> np.ndarray:
    """fp16 bits of u_n * max|W[n,:]| / 448, u_n ~ U[0.5, 2] (cfg2's recipe)."""
    u = g.uniform(0.5, 2.0, size=w_f32.shape[0]).astype(np.float32)
    s = u * np.abs(w_f32).max(axis=1) / np.float32(448.0)
    s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    return f32_to_f16_bits(s)


def int4_weight(g: np.random.Generator, N: int, K: int) -> np.ndarray:
    """int values in [-8, 7] (unpacked), shape [N, K]."""
    return g.integers(-8, 8, size=(N, K), dtype=np.int8)


def w4a8_channel_scales(g: np.random.Generator, N: int) -> np.ndarray:
    s = g.uniform(0.5, 2.0, size=N).astype(np.float32) * np.float32(2.0 ** -8)
    return f32_to_f16_bits(s)


def norm_weight(g: np.random.Generator, K: int, dtype: str) -> np.ndarray:
    """RMSNorm gain g[k] ~ U[0.5, 1.5] as fp16/bf16 bits [K] (synthetic: the
    pages give no trained values)."""
    return to_bits(g.uniform(0.5, 1.5, size=K).astype(np.float32), dtype)


def sample_rows(g: np.random.Generator, M: int, count: int) -> np.ndarray:
    """Sorted distinct row indices for spot-checking large outputs."""
    if count >= M:
        return np.arange(M, dtype=np.int64)
    return np.sort(g.choice(M, size=count, replace=False)).astype(np.int64)
