"""The whole low-bit linear layer on the CPU: quantize, decode-multiply, epilogue.

Test infrastructure (see the package docstring).  Composes ``quant``, ``gemm``
and ``epilogue`` in the order the layer runs them (page "How fal made Ideogram
V4 6x faster", paragraphs 2-4): activations quantized on the fly, the big GEMM
against quantized weights, the small op applied to the accumulator before the
one store.
"""
from __future__ import annotations

import numpy as np

from . import epilogue, gemm, quant


def quantize_operands(x_bits, w_bits, fmt: str):
    if fmt == "fp4":
        return quant.quantize_fp4(x_bits), quant.quantize_fp4(w_bits)
    if fmt == "fp8":
        return quant.quantize_fp8(x_bits), quant.quantize_fp8(w_bits)
    if fmt == "mx8":
        return quant.quantize_mx8(x_bits), quant.quantize_mx8(w_bits)
    if fmt == "nv4":
        return quant.quantize_nv4(x_bits), quant.quantize_nv4(w_bits)
    raise ValueError(fmt)


def accumulate(a, w, fmt: str, rows=None) -> np.ndarray:
    if fmt == "fp4":
        return gemm.gemm_fp4(a[0], a[1], w[0], w[1], rows=rows)
    if fmt == "mx8":
        return gemm.gemm_mx8(a[0], a[1], w[0], w[1], rows=rows)
    if fmt == "nv4":
        return gemm.gemm_nv4(a[0], a[1], a[2], w[0], w[1], w[2], rows=rows)
    return gemm.gemm_fp8(a[0], a[1], w[0], w[1], rows=rows)


def forward(x_bits, w_bits, fmt: str, epi: str, rows=None, **epi_kw) -> np.ndarray:
    """float64 output of the layer (before the bf16 store) for all rows or the given rows."""
    a, w = quantize_operands(x_bits, w_bits, fmt)
    if epi == "gate_residual":
        epi_kw = dict(epi_kw, row_ids=rows)
    return epilogue.apply(epi, accumulate(a, w, fmt, rows=rows), **epi_kw)
