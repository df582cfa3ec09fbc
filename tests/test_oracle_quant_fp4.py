"""Pins of the oracle's FP4 E2M1 / E8M0 block-32 quantizer.

* exhaustive agreement of two independent rounding rules over every finite bf16
  value at every scale byte;
* hand-derived worked examples (tests/golden/fp4_worked_examples.txt);
* exact round trips of values on the grid and the half-gap error bound.
"""
import numpy as np
import pytest

from oracle import formats, quant
from tests.conftest import read_golden


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = formats.bf16_to_f64(bits)
    keep = np.isfinite(x)
    return bits[keep], x[keep]


def test_rounding_rules_agree_for_every_bf16_and_every_scale_byte():
    bits, x = _all_finite_bf16()
    sign = ((bits >> 15) & 1).astype(np.uint8)
    for byte in range(0, 255):
        v = np.abs(x) * 2.0 ** (127 - byte)               # exact in float64
        a = quant.e2m1_rne_threshold(v)
        b = quant.e2m1_rne_bruteforce(v)
        assert np.array_equal(a, b), byte
        # the rounded magnitude is a nearest grid point
        g = formats.E2M1_GRID
        err = np.abs(g[a] - np.minimum(v, 6.0))
        assert np.all(err <= np.abs(v[:, None] - g).min(axis=1) + 0)
    assert sign.max() == 1


def test_scale_byte_rule():
    amax = np.array([7.0, 0.30078125, 1.0, 6.0, 8.0, 62.0, 0.0, 1.5 * 2.0 ** -125, 2.0 ** -133,
                     1.9921875 * 2.0 ** 127, 3.999, 4.0])
    exp = [127, 123, 125, 127, 128, 130, 0, 0, 0, 252, 126, 127]
    np.testing.assert_array_equal(quant.fp4_scale_byte(amax), exp)
    # the block maximum always lands in [4, 8) after scaling (or the byte clamps at 0)
    rng = np.random.default_rng(3)
    a = np.abs(rng.standard_normal(10000)) * 2.0 ** rng.integers(-100, 100, 10000)
    b = quant.fp4_scale_byte(a).astype(np.int64)
    v = a * 2.0 ** (127 - b)
    assert np.all((v >= 4) & (v < 8))


@pytest.mark.parametrize("row", read_golden("fp4_worked_examples.txt"), ids=lambda r: r[0])
def test_worked_examples(row):
    name, vals, byte, codes, first = row
    bits = np.zeros((1, 32), dtype=np.uint16)
    v = [int(t, 16) for t in vals.split()]
    bits[0, :len(v)] = v
    packed, scales = quant.quantize_fp4(bits)
    assert int(scales[0, 0]) == int(byte)
    got = quant.unpack_fp4_codes(packed)[0, :len(v)]
    assert [int(c) for c in got] == [int(c, 16) for c in codes.split()]
    assert int(packed[0, 0]) == int(first, 16)
    # both rounding rules give the same codes
    p2, s2 = quant.quantize_fp4(bits, rounding=quant.e2m1_rne_bruteforce)
    assert np.array_equal(p2, packed) and np.array_equal(s2, scales)


def test_grid_values_round_trip_exactly():
    # every grid value * 2^e in a block whose maximum is 4*2^e or 6*2^e comes back unchanged
    for e in (-120, -7, 0, 3, 100):
        for top in (4.0, 6.0):
            for s in (1.0, -1.0):
                vals = np.concatenate([formats.E2M1_GRID, -formats.E2M1_GRID])[:, None] * 2.0 ** e * s
                blk = np.zeros((vals.size, 32))
                blk[:, 0] = top * 2.0 ** e
                blk[:, 1] = vals[:, 0]
                bits = (blk.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
                assert np.array_equal(formats.bf16_to_f64(bits), blk)
                packed, scales = quant.quantize_fp4(bits)
                deq = quant.dequantize_fp4(packed, scales)
                np.testing.assert_array_equal(deq, blk)


def test_error_bound_on_random_blocks():
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(0)
    x = rng.standard_normal((256, 256)).astype(np.float32) * np.float32(3.0)
    x[:, 7] *= 20
    bits = f32_to_bf16_bits(x)
    packed, scales = quant.quantize_fp4(bits)
    deq = quant.dequantize_fp4(packed, scales)
    xv = formats.bf16_to_f64(bits)
    X = formats.e8m0_decode(scales).repeat(32, axis=1)
    a = np.abs(xv) / X
    # half the local grid gap below 6; the clip distance above 6
    gap = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    bound = np.where(a <= 6, gap / 2, a - 6) * X
    assert np.all(np.abs(deq - xv) <= bound)


def test_sign_is_kept_and_nibbles_are_low_first():
    bits = np.zeros((1, 64), dtype=np.uint16)
    bits[0, 0] = 0xBD00          # -0.03125: rounds to magnitude 0 in a block of max 1
    bits[0, 1] = 0x3F80          # 1.0
    packed, scales = quant.quantize_fp4(bits)
    assert packed[0, 0] == (0x8 | (0x6 << 4))
    assert scales[0, 1] == 0 and np.all(packed[0, 16:] == 0)


def test_non_finite_input_is_rejected():
    bits = np.zeros((1, 32), dtype=np.uint16)
    bits[0, 3] = 0x7F80
    with pytest.raises(ValueError):
        quant.quantize_fp4(bits)
