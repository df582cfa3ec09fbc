"""Epilogues applied to the float64 accumulator before the single store (CPU oracle).

Test infrastructure (see the package docstring).

Page "How fal made Ideogram V4 6x faster" (news.ditty.ir):
* paragraph 3 -- the small op after a big GEMM (RMSNorm, gated-SiLU) is applied
  right before the result is stored, so the output reaches HBM once; per-head
  RMSNorm, with head_dim 256 handled by a revisit schedule (a schedule only: the
  mathematics is the same as for any head size, so the oracle has no schedule);
* paragraph 4 -- gated-SiLU: C = A @ B, output = SiLU(C[:, :N//2]) * C[:, N//2:].

Two more small ops of a DiT block in the same place: the GELU of an MLP (page on
Google's on-device diffusion work (laaro.com), fused GELU kernels; FLUX-style MLPs
use its tanh form), and the gated residual update of adaLN-style blocks, the
small op after the attention-output and MLP-down projections.

Readings where the pages are silent: GELU-tanh(x) = 0.5 x (1 + tanh(sqrt(2/pi)
(x + 0.044715 x^3))); the gated residual is out[m, n] = residual[m, n] +
gate[m // rows_per_gate, n] * C[m, n], one gate row per sample of rows_per_gate
tokens, residual in bf16, gate in fp32; SiLU(x) = x / (1 + exp(-x)); RMSNorm is the
textbook y = x / sqrt(mean_d(x^2) + eps) * gamma[d], with the mean over the head
dimension, eps inside the square root, one gamma per head-dimension element shared
by all heads, separate gammas for the Q and K heads, and the GEMM columns ordered
[Q | K | V], head-major.  V columns pass through unchanged.  The epilogue acts on
the un-rounded accumulator: the fused kernel never rounds C before the small op.
"""
from __future__ import annotations

import math

import numpy as np

from . import formats


def identity(acc: np.ndarray) -> np.ndarray:
    return np.asarray(acc, dtype=np.float64)


def silu(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))           # -> -0.0 for very negative x, never NaN


GELU_TANH_C = 0.044715
SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        return 0.5 * x * (1.0 + np.tanh(SQRT_2_OVER_PI * (x + GELU_TANH_C * x ** 3)))


def gate_residual(acc: np.ndarray, residual_bits, gate, rows_per_gate: int, row_ids=None) -> np.ndarray:
    """residual + gate * acc for the accumulator rows ``row_ids`` (all rows if None):
    row m takes residual row m (bf16 bits, [M, N]) and gate row m // rows_per_gate
    (fp32, [ceil(M / rows_per_gate), N])."""
    acc = np.asarray(acc, dtype=np.float64)
    ids = np.arange(acc.shape[0]) if row_ids is None else np.asarray(row_ids)
    res = formats.bf16_to_f64(np.asarray(residual_bits, dtype=np.uint16)[ids])
    g = np.asarray(gate, dtype=np.float32).astype(np.float64)[ids // rows_per_gate]
    return res + g * acc


def gated_silu(acc: np.ndarray) -> np.ndarray:
    acc = np.asarray(acc, dtype=np.float64)
    n = acc.shape[1]
    if n % 2:
        raise ValueError("gated-SiLU needs an even GEMM width")
    return silu(acc[:, : n // 2]) * acc[:, n // 2:]


def qk_rmsnorm(acc: np.ndarray, n_heads: int, head_dim: int, gamma_q, gamma_k, eps: float) -> np.ndarray:
    acc = np.asarray(acc, dtype=np.float64)
    M, N = acc.shape
    H, D = n_heads, head_dim
    if N != 3 * H * D:
        raise ValueError("QK-RMSNorm expects N == 3 * n_heads * head_dim ([Q | K | V])")
    out = acc.copy()
    for part, gamma in ((0, gamma_q), (1, gamma_k)):
        x = acc[:, part * H * D:(part + 1) * H * D].reshape(M, H, D)
        ms = np.mean(x * x, axis=-1, keepdims=True)
        y = x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)
        out[:, part * H * D:(part + 1) * H * D] = y.reshape(M, H * D)
    return out


def apply(epi: str, acc: np.ndarray, **kw) -> np.ndarray:
    if epi == "identity":
        return identity(acc)
    if epi == "gated_silu":
        return gated_silu(acc)
    if epi == "qk_rmsnorm":
        return qk_rmsnorm(acc, kw["n_heads"], kw["head_dim"], kw["gamma_q"], kw["gamma_k"], kw["eps"])
    if epi == "gelu_tanh":
        return gelu_tanh(acc)
    if epi == "gate_residual":
        return gate_residual(acc, kw["residual"], kw["gate"], kw["rows_per_gate"], kw.get("row_ids"))
    raise ValueError(epi)
