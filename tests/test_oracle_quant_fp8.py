"""Pins of the oracle's FP8 E4M3 row-scaled quantizer.

* two independent E4M3 rounding rules agree on every rounding class of fp32
  (sign x exponent x the four leading mantissa bits x sticky patterns) and on
  random values;
* hand-derived worked examples (tests/golden/fp8_worked_examples.txt), with the
  per-row scale also recomputed in exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats, quant
from tests.conftest import read_golden


def _rounding_classes():
    out = []
    for s in (0, 1):
        for e in range(0, 255):
            for top in range(16):
                for low in (0, 1, 0x3FFFF, 0x40000, 0x40001, 0x7FFFF):
                    out.append((s << 31) | (e << 23) | (top << 19) | low)
    return np.array(out, dtype=np.uint32).view(np.float32)


def test_rounding_rules_agree_on_all_rounding_classes():
    y = _rounding_classes()
    np.testing.assert_array_equal(quant.e4m3_rne_fields(y), quant.e4m3_rne_bruteforce(y))


def test_rounding_rules_agree_on_random_values():
    rng = np.random.default_rng(1)
    y = (rng.standard_normal(2_000_000) * 2.0 ** rng.integers(-12, 9, 2_000_000)).astype(np.float32)
    np.testing.assert_array_equal(quant.e4m3_rne_fields(y), quant.e4m3_rne_bruteforce(y))


def test_rounding_is_nearest():
    y = _rounding_classes()
    y = y[np.abs(y) <= 448]
    c = quant.e4m3_rne_fields(y)
    d = formats.e4m3_decode(c)
    err = np.abs(d - y.astype(np.float64))
    best = np.abs(np.abs(y.astype(np.float64))[:, None] - formats.E4M3_POS[None, :]).min(axis=1)
    np.testing.assert_array_equal(err, best)


@pytest.mark.parametrize("row", [r for r in read_golden("fp8_worked_examples.txt") if r[0] == "element"],
                         ids=lambda r: r[1])
def test_element_examples(row):
    _, val, code = row
    y = np.array([float(val)], dtype=np.float32)
    assert int(quant.e4m3_rne_fields(y)[0]) == int(code, 16)
    assert int(quant.e4m3_rne_bruteforce(y)[0]) == int(code, 16)


def _rn32(q: Fraction) -> float:
    """Round a rational to the nearest fp32 (ties to even), exactly."""
    f = float(q)                      # correctly rounded to float64 ...
    cand = np.float32(f)
    best = None
    for c in (np.nextafter(cand, np.float32(-np.inf)), cand, np.nextafter(cand, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - q)
        key = (d, int(np.array(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


@pytest.mark.parametrize("row", [r for r in read_golden("fp8_worked_examples.txt") if r[0] == "row"],
                         ids=lambda r: r[1])
def test_row_examples(row):
    _, vals, scale, codes = row
    bits = np.array([[int(t, 16) for t in vals.split()]], dtype=np.uint16)
    c, s = quant.quantize_fp8(bits)
    assert float(s[0]) == float(scale)
    assert [int(v) for v in c[0]] == [int(t, 16) for t in codes.split()]


def test_row_scale_matches_exact_rational_division():
    rng = np.random.default_rng(2)
    from workloads import f32_to_bf16_bits
    x = f32_to_bf16_bits(rng.standard_normal((64, 96)).astype(np.float32) * 5)
    c, s = quant.quantize_fp8(x)
    xv = formats.bf16_to_f64(x)
    for r in range(0, 64, 7):
        amax = Fraction(float(np.abs(xv[r]).max()))
        s_ref = _rn32(amax / 448)
        assert np.float32(s[r]) == s_ref
        for k in range(0, 96, 11):
            y = _rn32(Fraction(float(xv[r, k])) / Fraction(float(s_ref)))
            assert c[r, k] == quant.e4m3_rne_bruteforce(np.array([y], np.float32))[0]


@pytest.mark.parametrize("amax_bits", [0x3FC4, 0x40C4])
def test_every_bf16_below_row_max_matches_exact_division(amax_bits):
    """One row holding every non-negative bf16 value up to its maximum.  For these
    maxima, x * fl32(1 / s) and fl32(x / s) land on opposite sides of an E4M3
    rounding boundary for some elements, so a reciprocal-multiply quantizer fails."""
    bits = np.arange(0, amax_bits + 1, dtype=np.uint16)[None, :]
    c, s = quant.quantize_fp8(bits)
    s_ref = _rn32(Fraction(float(formats.bf16_to_f64(np.uint16(amax_bits)))) / 448)
    assert np.float32(s[0]) == s_ref
    xv = formats.bf16_to_f64(bits[0])
    y = np.array([_rn32(Fraction(float(v)) / Fraction(float(s_ref))) for v in xv], dtype=np.float32)
    assert np.array_equal(c[0], quant.e4m3_rne_bruteforce(y))


def test_row_quantization_error_bound():
    rng = np.random.default_rng(4)
    from workloads import f32_to_bf16_bits
    x = f32_to_bf16_bits(rng.standard_normal((128, 512)).astype(np.float32))
    c, s = quant.quantize_fp8(x)
    xv = formats.bf16_to_f64(x)
    deq = quant.dequantize_fp8(c, s)
    # 3 mantissa bits: relative error <= 2^-4 in the normal range, absolute <= 2^-10*s below it
    y = np.abs(xv) / s[:, None]
    bound = np.where(y >= 2.0 ** -6, np.abs(xv) * 2.0 ** -4 * (1 + 1e-6), 2.0 ** -10 * s[:, None])
    assert np.all(np.abs(deq - xv) <= bound + 1e-30)
