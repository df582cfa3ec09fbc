"""Epilogues applied to the float64 accumulator before the single store (CPU oracle).

Test infrastructure (see the package docstring).

Page "How fal made Ideogram V4 6x faster" (news.ditty.ir):
* paragraph 3 -- the small op after a big GEMM (RMSNorm, gated-SiLU) is applied
  right before the result is stored, so the output reaches HBM once; per-head
  RMSNorm, with head_dim 256 handled by a revisit schedule (a schedule only: the
  mathematics is the same as for any head size, so the oracle has no schedule);
* paragraph 4 -- gated-SiLU: C = A @ B, output = SiLU(C[:, :N//2]) * C[:, N//2:].

Readings where the pages are silent: SiLU(x) = x / (1 + exp(-x)); RMSNorm is the
textbook y = x / sqrt(mean_d(x^2) + eps) * gamma[d], with the mean over the head
dimension, eps inside the square root, one gamma per head-dimension element shared
by all heads, separate gammas for the Q and K heads, and the GEMM columns ordered
[Q | K | V], head-major.  V columns pass through unchanged.  The epilogue acts on
the un-rounded accumulator: the fused kernel never rounds C before the small op.
"""
from __future__ import annotations

import numpy as np


def identity(acc: np.ndarray) -> np.ndarray:
    return np.asarray(acc, dtype=np.float64)


def silu(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))           # -> -0.0 for very negative x, never NaN


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
    raise ValueError(epi)
