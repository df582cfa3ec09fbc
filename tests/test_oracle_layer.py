"""Pins of the oracle's layer composition (``oracle.layer``).

``layer.forward`` chains the pieces every GPU parity test compares against:
quantize activations and weights on the fly, multiply in float64, apply the small
op to the un-rounded accumulator (page "How fal made Ideogram V4 6x faster",
paragraphs 2-4).  Each piece is pinned on its own elsewhere; these tests pin the
composition.  For every format and epilogue a tiny problem is recomputed here
without ``oracle.layer``, ``oracle.gemm`` or ``oracle.epilogue``:

* the codes and scales come from the (separately pinned) quantizers, applied to
  the activation rows and to the weight rows alike;
* every code is decoded element by element from its bit fields into an exact
  ``fractions.Fraction`` and the dot products are summed exactly, with the FP8
  row scale of the activation row and the column scale of the weight row, or
  the two NVFP4 tensor scales;
* the epilogue is written out per element with ``math``.

FP4 sums are exact in float64, so the identity epilogue must agree bit for bit;
the other cases agree to 2**-40 relative.  A slip in the composition -- the wrong
quantizer for W, the activation and weight scales paired the wrong way round, a
dropped ``row_ids`` on a row subset of the gated residual -- fails here.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import layer, quant
from workloads import f32_to_bf16_bits

FORMATS = ["fp4", "fp8", "mx8", "nv4"]
EPIS = ["identity", "gated_silu", "qk_rmsnorm", "gelu_tanh", "gate_residual"]
M, K = 3, 64
N_PLAIN = 16                   # identity, GELU, gated residual; gated-SiLU: 8 pairs
H, D = 1, 8                    # QK-RMSNorm: N = 3 * H * D = 24 (head size is free in the oracle)
RPG = 2                        # gated residual: tokens per gate row
REL = 2.0 ** -40

E2M1_MAG = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
            Fraction(6)]


def e2m1(code: int) -> Fraction:
    v = E2M1_MAG[code & 7]
    return -v if code & 8 else v


def e4m3(code: int) -> Fraction:
    """OCP E4M3 from its fields: 1 sign, 4 exponent (bias 7), 3 mantissa bits."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    assert not (e == 15 and m == 7), "NaN code"
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def e8m0(byte: int) -> Fraction:
    assert byte != 255
    return Fraction(2) ** (int(byte) - 127)


def nibble(packed: np.ndarray, r: int, k: int) -> int:
    b = int(packed[r, k // 2])
    return b & 0xF if k % 2 == 0 else b >> 4


def decode_exact(fmt: str, q, r: int, k: int) -> Fraction:
    """Element (r, k) of a quantized operand as an exact rational (FP8 row/column and
    NVFP4 tensor scales excluded: they are applied to the whole dot product)."""
    if fmt == "fp4":
        codes, scales = q
        return e2m1(nibble(codes, r, k)) * e8m0(scales[r, k // 32])
    if fmt == "fp8":
        codes, _ = q
        return e4m3(int(codes[r, k]))
    if fmt == "mx8":
        codes, scales = q
        return e4m3(int(codes[r, k])) * e8m0(scales[r, k // 32])
    codes, scales, _ = q
    return e2m1(nibble(codes, r, k)) * e4m3(int(scales[r, k // 16]))


def quantizer(fmt: str):
    return {"fp4": quant.quantize_fp4, "fp8": quant.quantize_fp8, "mx8": quant.quantize_mx8,
            "nv4": quant.quantize_nv4}[fmt]


def exact_accumulator(fmt: str, x_bits, w_bits):
    """Exact C = A W^T of the quantized operands, [M][N] Fractions."""
    qa, qw = quantizer(fmt)(x_bits), quantizer(fmt)(w_bits)
    rows, cols = x_bits.shape[0], w_bits.shape[0]
    acc = []
    for m in range(rows):
        a = [decode_exact(fmt, qa, m, k) for k in range(K)]
        row = []
        for n in range(cols):
            s = sum((a[k] * decode_exact(fmt, qw, n, k) for k in range(K)), Fraction(0))
            if fmt == "fp8":
                s *= Fraction(float(qa[1][m])) * Fraction(float(qw[1][n]))
            elif fmt == "nv4":
                s *= Fraction(float(qa[2])) * Fraction(float(qw[2]))
            row.append(s)
        acc.append(row)
    return acc


def silu(v: float) -> float:
    return v / (1.0 + math.exp(-v)) if v > -700 else -0.0


def gelu_tanh(v: float) -> float:
    return 0.5 * v * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (v + 0.044715 * v ** 3)))


def bf16_value(bits: int) -> float:
    return float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0])


def expected(epi: str, acc, inp) -> np.ndarray:
    """The small op per element, from the exact accumulator rows (all M rows)."""
    c = [[float(v) for v in row] for row in acc]
    rows, cols = len(c), len(c[0])
    if epi == "identity":
        return np.array(c)
    if epi == "gelu_tanh":
        return np.array([[gelu_tanh(v) for v in row] for row in c])
    if epi == "gated_silu":
        half = cols // 2
        return np.array([[silu(row[j]) * row[j + half] for j in range(half)] for row in c])
    if epi == "gate_residual":
        out = np.empty((rows, cols))
        for m in range(rows):
            for n in range(cols):
                out[m, n] = bf16_value(inp["residual"][m, n]) + float(inp["gate"][m // RPG, n]) * c[m][n]
        return out
    out = np.array(c)
    for m in range(rows):
        for part, gamma in ((0, inp["gamma_q"]), (1, inp["gamma_k"])):
            for h in range(H):
                c0 = part * H * D + h * D
                ms = sum(c[m][c0 + d] ** 2 for d in range(D)) / D
                inv = 1.0 / math.sqrt(ms + inp["eps"])
                for d in range(D):
                    out[m, c0 + d] = c[m][c0 + d] * inv * float(gamma[d])
    return out


def make_case(fmt: str, epi: str, seed: int) -> dict:
    rng = np.random.default_rng(seed)
    n = 3 * H * D if epi == "qk_rmsnorm" else N_PLAIN
    # a few binades of spread, so that block scales differ along K and across rows
    x = rng.standard_normal((M, K)).astype(np.float32) * np.float32(2.0) ** rng.integers(-3, 4, (M, 1))
    x[:, 5] *= 20.0                                            # one outlier channel
    w = (rng.standard_normal((n, K)) / math.sqrt(K)).astype(np.float32)
    w *= np.float32(2.0) ** rng.integers(-2, 3, (n, 1))
    inp = {"x": f32_to_bf16_bits(x), "w": f32_to_bf16_bits(w), "eps": 1e-6}
    if epi == "qk_rmsnorm":
        inp["gamma_q"] = rng.uniform(0.5, 1.5, D).astype(np.float32)
        inp["gamma_k"] = rng.uniform(0.5, 1.5, D).astype(np.float32)
    if epi == "gate_residual":
        inp["residual"] = f32_to_bf16_bits(rng.standard_normal((M, n)).astype(np.float32))
        inp["gate"] = (rng.standard_normal(((M + RPG - 1) // RPG, n)) * 0.5).astype(np.float32)
    return inp


def epi_kwargs(epi: str, inp: dict) -> dict:
    if epi == "qk_rmsnorm":
        return dict(n_heads=H, head_dim=D, gamma_q=inp["gamma_q"], gamma_k=inp["gamma_k"], eps=inp["eps"])
    if epi == "gate_residual":
        return dict(residual=inp["residual"], gate=inp["gate"], rows_per_gate=RPG)
    return {}


def assert_close(got: np.ndarray, want: np.ndarray, exact: bool, label: str):
    assert got.shape == want.shape, (label, got.shape, want.shape)
    if exact:
        np.testing.assert_array_equal(got, want, err_msg=label)
        return
    scale = np.max(np.abs(want), axis=1, keepdims=True)
    err = np.abs(got - want)
    assert np.all(err <= REL * scale + 1e-300), f"{label}: max rel err {float((err / scale).max()):.3g}"


CASES = [(f, e) for f in FORMATS for e in EPIS]


@pytest.mark.parametrize("fmt,epi", CASES, ids=[f"{f}-{e}" for f, e in CASES])
def test_forward_equals_exact_composition(fmt, epi):
    inp = make_case(fmt, epi, seed=FORMATS.index(fmt) * 10 + EPIS.index(epi))
    acc = exact_accumulator(fmt, inp["x"], inp["w"])
    want = expected(epi, acc, inp)
    got = layer.forward(inp["x"], inp["w"], fmt, epi, **epi_kwargs(epi, inp))
    assert_close(got, want, exact=(fmt == "fp4" and epi == "identity"), label=f"{fmt}/{epi}")


@pytest.mark.parametrize("fmt,epi", CASES, ids=[f"{f}-{e}" for f, e in CASES])
def test_forward_on_row_subsets(fmt, epi):
    """``rows=`` (the sampled-row path of the largest-size tests) gives exactly those
    rows of the full computation, in the order asked for; for the gated residual
    each row takes its own residual row and its sample's gate row."""
    inp = make_case(fmt, epi, seed=100 + FORMATS.index(fmt) * 10 + EPIS.index(epi))
    rows = np.array([2, 0])                       # row 2 sits in the second gate sample
    acc = exact_accumulator(fmt, inp["x"], inp["w"])
    want = expected(epi, acc, inp)[rows]
    got = layer.forward(inp["x"], inp["w"], fmt, epi, rows=rows, **epi_kwargs(epi, inp))
    assert_close(got, want, exact=(fmt == "fp4" and epi == "identity"), label=f"{fmt}/{epi} rows {rows}")


def test_quantize_operands_uses_one_format_for_both():
    """The activations and the weights are quantized by the same rule (the weight
    packer applies the activation rule along K to every weight row)."""
    inp = make_case("fp4", "identity", seed=7)
    for fmt in FORMATS:
        a, w = layer.quantize_operands(inp["x"], inp["w"], fmt)
        qa, qw = quantizer(fmt)(inp["x"]), quantizer(fmt)(inp["w"])
        for got, want in ((a, qa), (w, qw)):
            assert len(got) == len(want)
            for g, e in zip(got, want):
                np.testing.assert_array_equal(np.asarray(g), np.asarray(e), err_msg=fmt)
