"""Roofline arithmetic for the W4A4 group-quantized GEMM on MI355X.

The crossover model is the one the blog page "Why INT4 Weight-Only Quantization
Doesn't Speed Up Prefill" works through (its code block on where a
weight-stationary GEMM stops being memory-bound): a GEMM that reads a [K, N]
weight of ``b`` bytes per element once for ``B`` tokens does 2*B*K*N FLOP on
K*N*b bytes, so its intensity is 2B/b and it turns compute-bound at
B = ridge * b / 2 with ridge = peak FLOP/s over HBM bytes/s.

For W4A4 the per-call work and traffic are
    ops   = 2*M*N*K
    bytes = M*K/2 + 4*M*K/g_a + N*K/2 + 4*N*K/g_w + 2*M*N
(packed activations + their fp32 scales, packed weights + scales, fp16 output).
"""
from __future__ import annotations

# MI355X published peaks (dense, no sparsity)
PEAK_INT8_OPS = 5.0e15        # int8 MFMA, ops/s
PEAK_FP8_FLOPS = 5.0e15
PEAK_FP6_FLOPS = 10.1e15      # fp6 / fp4 MFMA, dense
PEAK_BF16_FLOPS = 2.5e15
PEAK_FP32_VECTOR_FLOPS = 157.3e12
PEAK_HBM_BYTES = 8.0e12       # HBM3E, bytes/s


def crossover(peak_flops: float, hbm_bytes_per_s: float, bytes_per_weight: float) -> float:
    """Concurrent tokens at which a weight-stationary GEMM becomes compute-bound."""
    ridge = peak_flops / hbm_bytes_per_s
    return ridge * bytes_per_weight / 2.0


def gemm_ops(M: int, N: int, K: int) -> float:
    return 2.0 * M * N * K


def gemm_bytes(M: int, N: int, K: int, ga: int, gw: int) -> float:
    """Algorithmic HBM bytes of one W4A4 GEMM call (each operand read once)."""
    return M * K / 2 + 4.0 * M * K / ga + N * K / 2 + 4.0 * N * K / gw + 2.0 * M * N


def quantize_bytes(M: int, K: int, g: int) -> float:
    """Algorithmic HBM bytes of one activation quantization (fp16 in, packed + scales out)."""
    return 2.0 * M * K + M * K / 2 + 4.0 * M * K / g


def bound_of(M: int, N: int, K: int, ga: int, gw: int) -> str:
    """'mfma' when the call's intensity is past the int8 MFMA / HBM ridge, else 'hbm'."""
    intensity = gemm_ops(M, N, K) / gemm_bytes(M, N, K, ga, gw)
    return "mfma" if intensity >= PEAK_INT8_OPS / PEAK_HBM_BYTES else "hbm"
