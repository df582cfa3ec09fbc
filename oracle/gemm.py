"""Decode-then-multiply GEMM of the low-bit linear layer (CPU oracle, float64).

Test infrastructure (see the package docstring).

The product is C = A @ B with A the quantized activations [M, K] and B the
quantized weights, given in torch Linear layout W [N, K] (so C = A W^T); page
"How fal made Ideogram V4 6x faster", paragraph 4 (C = A @ B).

FP4: acc[m, n] = sum_k dec(a)[m, k] * dec(w)[n, k], every operand an E2M1 value
times its block's E8M0 scale.  Decoded E2M1 values are integers <= 12 times
2**-1, so every product is an integer times a power of two and every block sum is
an integer < 2**13 times a power of two; float64 holds the whole sum exactly as
long as the spread of block exponents in a row/column pair stays small.
``fp4_sum_is_exact`` checks the sufficient condition, so the result below is the
exact rational value regardless of the summation order a BLAS picks.

FP8: acc[m, n] = (sum_k e4m3(a)[m, k] * e4m3(w)[n, k]) * s_a[m] * s_w[n].  Every
E4M3 value is a multiple of 2**-9 below 2**9, so every product is a multiple of
2**-18 below 2**18 and a sum of K <= 2**14 of them fits in 50 bits: the sum is
exact in float64; the two scale multiplications round once each (~1e-16).

MXFP8: acc[m, n] = sum_k dec(a)[m, k] * dec(w)[n, k], every operand an E4M3 value
times its block's E8M0 scale.  A product spans up to 36 significant bits, so
blocks with different scales need not sum exactly in float64; the float64 sum is
within K * 2**-53 * sum_k |a_k w_k| of the exact value (below 1e-12 relative to
the sum of magnitudes for K <= 16384), many orders of magnitude under any fp32
accumulation or bf16 storage error the layer makes.

NVFP4: acc[m, n] = (sum_k e2m1(a) s_b(a) e2m1(w) s_b(w)) * s_t(A) * s_t(W), the
block-scaled products summed in float64 (the same bound as MXFP8), then the two
tensor scales.
"""
from __future__ import annotations

import math

import numpy as np

from . import formats, quant

ROW_CHUNK = 1024


def fp4_sum_is_exact(a_scales: np.ndarray, w_scales: np.ndarray, K: int) -> bool:
    """Sufficient condition for float64 exactness of every FP4 dot product.

    In units of the smallest possible product, a product is at most 144 * 2**d
    where d = (ea + ew) - min(ea + ew) over the non-zero blocks of the pair, and
    there are K products.  Exact if K * 144 * 2**(max spread) < 2**53.
    """
    def spread(s):
        s = np.asarray(s, dtype=np.int64)
        nz = s > 0
        hi = np.where(nz, s, -1).max(axis=1)
        lo = np.where(nz, s, 1 << 20).min(axis=1)
        sp = np.where(hi >= 0, hi - lo, 0)
        return int(sp.max()) if sp.size else 0
    bits = spread(a_scales) + spread(w_scales) + math.log2(144) + math.log2(max(K, 1))
    return bits < 53


def gemm_fp4(a_codes, a_scales, w_codes, w_scales, rows=None) -> np.ndarray:
    """acc = dequant(A) @ dequant(W)^T in float64, [M, N] (or the chosen rows of A)."""
    K = np.asarray(a_codes).shape[1] * 2
    if not fp4_sum_is_exact(a_scales, w_scales, K):
        raise ArithmeticError("block exponent spread too wide for an exact float64 sum")
    Wd = quant.dequantize_fp4(w_codes, w_scales)
    sel = np.arange(np.asarray(a_codes).shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((sel.size, Wd.shape[0]), dtype=np.float64)
    for i in range(0, sel.size, ROW_CHUNK):
        r = sel[i:i + ROW_CHUNK]
        Ad = quant.dequantize_fp4(np.asarray(a_codes)[r], np.asarray(a_scales)[r])
        out[i:i + ROW_CHUNK] = Ad @ Wd.T
    return out


def gemm_fp8(a_codes, a_scales, w_codes, w_scales, rows=None) -> np.ndarray:
    """acc = (e4m3(A) @ e4m3(W)^T) * s_a[:, None] * s_w[None, :] in float64."""
    Wd = formats.e4m3_decode(w_codes)
    sw = np.asarray(w_scales, dtype=np.float64)
    sel = np.arange(np.asarray(a_codes).shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((sel.size, Wd.shape[0]), dtype=np.float64)
    for i in range(0, sel.size, ROW_CHUNK):
        r = sel[i:i + ROW_CHUNK]
        Ad = formats.e4m3_decode(np.asarray(a_codes)[r])
        sa = np.asarray(a_scales, dtype=np.float64)[r]
        out[i:i + ROW_CHUNK] = (Ad @ Wd.T) * sa[:, None] * sw[None, :]
    return out


def gemm_mx8(a_codes, a_scales, w_codes, w_scales, rows=None) -> np.ndarray:
    """acc = dequant(A) @ dequant(W)^T in float64, MXFP8 operands, [M, N] (or the chosen rows)."""
    Wd = quant.dequantize_mx8(w_codes, w_scales)
    sel = np.arange(np.asarray(a_codes).shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((sel.size, Wd.shape[0]), dtype=np.float64)
    for i in range(0, sel.size, ROW_CHUNK):
        r = sel[i:i + ROW_CHUNK]
        Ad = quant.dequantize_mx8(np.asarray(a_codes)[r], np.asarray(a_scales)[r])
        out[i:i + ROW_CHUNK] = Ad @ Wd.T
    return out


def gemm_nv4(a_codes, a_scales, a_st, w_codes, w_scales, w_st, rows=None) -> np.ndarray:
    """acc = (dequant(A) @ dequant(W)^T) in float64 with NVFP4 operands (tensor scales included)."""
    Wd = quant.dequantize_nv4(w_codes, w_scales, 1.0)
    sel = np.arange(np.asarray(a_codes).shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((sel.size, Wd.shape[0]), dtype=np.float64)
    st = float(np.float32(a_st)) * float(np.float32(w_st))
    for i in range(0, sel.size, ROW_CHUNK):
        r = sel[i:i + ROW_CHUNK]
        Ad = quant.dequantize_nv4(np.asarray(a_codes)[r], np.asarray(a_scales)[r], 1.0)
        out[i:i + ROW_CHUNK] = (Ad @ Wd.T) * st
    return out
