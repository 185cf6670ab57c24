"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no quantization, packing or GEMM), so both the HIP path
and the CPU oracle can consume what it makes without sharing any code.

Recipes (the workloads the APEX4 page evaluates on are LLaMA-2 layers; no
weights or datasets are used, these stand in for them):
  * weights W[N, K]: N(0, 0.02) drawn in fp32, rounded to fp16 (RNE);
  * activations X[M, K], one of
      - ``normal``:   N(0, 1);
      - ``outlier``:  N(0, 1) with round(0.01*K) fixed channels, the same for
        every token, multiplied by 20 (outliers that stay in fixed channels
        across tokens, as the OSC page's Abstract observes for LLM activations);
      - ``student_t``: Student-t with 3 degrees of freedom (heavy-tailed),
        clipped to the fp16 range;
  * random packed INT4 operands: uniform random bytes, so every nibble value
    (-8 included) occurs; with uniform random fp32 scales.
One generator ``numpy.random.default_rng(seed)`` draws X first, then W; the
outlier channels come from ``default_rng([seed, 1])``.
"""
from __future__ import annotations

import numpy as np

ACT_KINDS = ("normal", "outlier", "student_t")


def outlier_channels(K: int, seed: int) -> np.ndarray:
    n_out = int(round(0.01 * K))
    rng = np.random.default_rng([seed, 1])
    return np.sort(rng.choice(K, size=n_out, replace=False))


def activations(rng: np.random.Generator, M: int, K: int, kind: str, seed: int) -> np.ndarray:
    if kind == "normal":
        x = rng.standard_normal((M, K), dtype=np.float32)
    elif kind == "outlier":
        x = rng.standard_normal((M, K), dtype=np.float32)
        ch = outlier_channels(K, seed)
        x[:, ch] *= np.float32(20.0)
    elif kind == "student_t":
        x = rng.standard_t(3, size=(M, K))
        x = np.clip(x, -65504.0, 65504.0).astype(np.float32)
    else:
        raise ValueError(f"unknown activation kind {kind!r}; one of {ACT_KINDS}")
    return x.astype(np.float16)


def weights(rng: np.random.Generator, N: int, K: int, std: float = 0.02) -> np.ndarray:
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    return w.astype(np.float16)


def problem(M: int, N: int, K: int, seed: int = 0, act: str = "normal"):
    """(X fp16 [M,K], W fp16 [N,K]) drawn from one seeded generator, X first."""
    rng = np.random.default_rng(seed)
    x = activations(rng, M, K, act, seed)
    w = weights(rng, N, K)
    return x, w


def random_packed(rows: int, K: int, G: int, seed: int, scale_lo: float = 0.5,
                  scale_hi: float = 2.0):
    """Uniform random packed bytes [rows, K/2] and fp32 scales [rows, G]."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    s = rng.uniform(scale_lo, scale_hi, size=(rows, G)).astype(np.float32)
    return q, s
