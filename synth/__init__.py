"""Seeded synthetic inputs for the W4A16 workloads.

This module only draws random numbers and stores them in the input dtypes the
workloads name (fp32, fp16, bf16 bit patterns).  It holds none of the
quantization or matmul arithmetic: both the CPU oracle and the GPU path take
their inputs from here, and nothing else is shared between them.

Conventions
-----------
* ``N(0, s)`` means mean 0 and *standard deviation* s (the vLLM page's
  repro script draws ``normal_(mean=0.0, std=0.5)``).
* Every tensor comes from its own PCG64 stream,
  ``numpy.random.default_rng([0, config_id, shape_idx, tensor_id])``; the
  single-matmul case uses seed 0 as stated for it.
* bf16 tensors are returned as ``uint16`` bit patterns, rounded from fp32 with
  round-to-nearest-even (NaN never occurs: inputs are finite draws).
"""

from __future__ import annotations

import numpy as np

# tensor ids inside one (config, shape) stream family
T_X = 0
T_W = 1
T_BIAS = 2
T_OUTLIER_MASK = 3
T_OUTLIER_VAL = 4
T_DY = 5
T_Q = 6  # separate Q/K/V weights for the fused-QKV operand
T_K = 7
T_V = 8


def rng(config_id: int, shape_idx: int, tensor_id: int) -> np.random.Generator:
    """Independent PCG64 stream per (config, shape, tensor)."""
    return np.random.default_rng([0, int(config_id), int(shape_idx), int(tensor_id)])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Store fp32 draws as bf16 (RNE).  Input generation only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(gen: np.random.Generator, shape, std: float) -> np.ndarray:
    """fp32 draws from N(0, std), generated in chunks to bound peak memory."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    chunk = 1 << 24
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        out[i:i + m] = gen.standard_normal(m, dtype=np.float32) * np.float32(std)
    return out.reshape(shape)


def activations_bf16(config_id: int, shape_idx: int, M: int, K: int, tensor_id: int = T_X) -> np.ndarray:
    """X (or dY) bf16 [M][K] ~ N(0, 1), as uint16 bits."""
    return f32_to_bf16_bits(normal(rng(config_id, shape_idx, tensor_id), (M, K), 1.0))


def weight(config_id: int, shape_idx: int, N: int, K: int, dtype: str, std: float = 0.02,
           tensor_id: int = T_W) -> np.ndarray:
    """W [N][K] ~ N(0, std) stored as 'f32' (float32), 'f16' (float16) or 'bf16' (uint16 bits)."""
    w = normal(rng(config_id, shape_idx, tensor_id), (N, K), std)
    if dtype == "f32":
        return w
    if dtype == "f16":
        return w.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(w)
    raise ValueError(dtype)


def weight_with_outliers(config_id: int, shape_idx: int, N: int, K: int, std: float = 0.02,
                         frac: float = 1e-3, outlier_std: float = 0.5) -> np.ndarray:
    """fp16 W ~ N(0, std) where an i.i.d. fraction ``frac`` of entries is replaced by N(0, outlier_std)."""
    w = normal(rng(config_id, shape_idx, T_W), (N, K), std)
    flat = w.reshape(-1)
    gmask = rng(config_id, shape_idx, T_OUTLIER_MASK)
    idx = np.flatnonzero(gmask.random(flat.size, dtype=np.float32) < np.float32(frac))
    vals = normal(rng(config_id, shape_idx, T_OUTLIER_VAL), (idx.size,), outlier_std)
    flat[idx] = vals
    return w.astype(np.float16)


def bias_f32(config_id: int, shape_idx: int, n: int, std: float = 0.1) -> np.ndarray:
    """fp32 bias ~ N(0, std)."""
    return normal(rng(config_id, shape_idx, T_BIAS), (n,), std)


def single_matmul_case():
    """The single W4A16 matmul workload: X bf16 [4][2048] ~ N(0,1), W fp32 [2048][2048] ~ N(0,0.02), seed 0.

    Both tensors come from one ``default_rng(0)`` stream (X first, then W).
    """
    g = np.random.default_rng(0)
    x = f32_to_bf16_bits(normal(g, (4, 2048), 1.0))
    w = normal(g, (2048, 2048), 0.02)
    return x, w
