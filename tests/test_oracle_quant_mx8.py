"""Pins of the oracle's MXFP8 quantizer (E4M3 elements, E8M0 scale per 32 K) and
of its decode-multiply GEMM.

* hand-derived worked examples (tests/golden/mx8_worked_examples.txt);
* the scale rule on every finite bf16 block maximum: the scaled maximum lands in
  [256, 512) unless the byte is clamped at 0;
* every code against a brute-force search of the scaled E4M3 grid, written from
  the definition (nearest grid point times the block scale, ties to the even code,
  saturation at 448 times the scale, the sign copied from x);
* exact round trip of blocks made of representable values, and the error bound
  of three mantissa bits;
* the GEMM against exact rational arithmetic on a small case, and (unit scales)
  against the FP8 GEMM's decode.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats, gemm, quant
from tests.conftest import read_golden
from workloads import f32_to_bf16_bits


@pytest.mark.parametrize("row", read_golden("mx8_worked_examples.txt"), ids=lambda r: r[1])
def test_block_examples(row):
    _, vals, byte, codes = row
    bits = np.zeros((1, 32), dtype=np.uint16)
    given = [int(t, 16) for t in vals.split()]
    bits[0, :len(given)] = given
    c, s = quant.quantize_mx8(bits)
    assert int(s[0, 0]) == int(byte)
    want = [int(t, 16) for t in codes.split()]
    assert [int(v) for v in c[0, :len(want)]] == want
    assert not c[0, len(want):].any()


def test_scale_rule_on_every_bf16_maximum():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)          # every finite non-negative bf16
    amax = formats.bf16_to_f64(bits)
    byte = quant.mx8_scale_byte(amax).astype(np.int64)
    scaled = amax * np.ldexp(1.0, 127 - byte)
    nz = amax > 0
    assert np.all(byte[~nz] == 0)
    inner = nz & (byte > 0)
    assert np.all((scaled[inner] >= 256) & (scaled[inner] < 512))
    clamped = nz & (byte == 0)
    assert np.all(scaled[clamped] < 512)                  # byte 0 is the smallest scale there is
    assert np.all(amax[clamped & (scaled < 256)] < 2.0 ** -119)
    assert byte.max() == 246                              # bf16's largest finite value, 2^127.99
    assert np.all(byte <= 254)


def _bruteforce_codes(xv, byte):
    """Per element: the signed E4M3 value times 2^(byte-127) nearest to x, ties to the
    even code; magnitudes past 448 * scale take 448 * scale."""
    scale = np.ldexp(1.0, int(byte) - 127)
    grid = formats.E4M3_POS * scale                      # index == magnitude code
    out = []
    for v in xv:
        a = min(abs(float(v)), 448.0 * scale)
        d = np.abs(grid - a)
        best = np.flatnonzero(d == d.min())
        code = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        sign = 1 if np.signbit(v) else 0
        out.append(code | (sign << 7))
    return out


def _blocks(rng, n):
    x = rng.standard_normal((n, 32)).astype(np.float32)
    x *= (2.0 ** rng.integers(-20, 20, (n, 1))).astype(np.float32)
    x[:, rng.integers(0, 32, n // 2)] *= 20.0                          # outliers
    x[rng.random((n, 32)) < 0.05] = 0.0
    x[rng.random((n, 32)) < 0.02] *= -0.0
    return f32_to_bf16_bits(x)


def test_codes_match_bruteforce_search():
    bits = _blocks(np.random.default_rng(5), 400)
    c, s = quant.quantize_mx8(bits)
    xv = formats.bf16_to_f64(bits)
    for r in range(bits.shape[0]):
        assert list(c[r]) == _bruteforce_codes(xv[r], s[r, 0]), r


def test_tiny_and_huge_blocks_match_bruteforce():
    """Blocks at the ends of the bf16 range: subnormal maxima (byte clamped to 0) and
    maxima near bf16's largest value, mixed with much smaller elements."""
    tiny = np.array([0x0001, 0x8003, 0x007F, 0x0080, 0x00FF, 0x0100, 0x8000] + [0] * 25, dtype=np.uint16)
    huge = np.array([0x7F7F, 0x7F00, 0xFEFF, 0x3F80, 0x0001, 0x4000] + [0] * 26, dtype=np.uint16)
    bits = np.stack([tiny, huge])
    c, s = quant.quantize_mx8(bits)
    xv = formats.bf16_to_f64(bits)
    assert int(s[0, 0]) == 0 and int(s[1, 0]) == 246
    for r in range(2):
        assert list(c[r]) == _bruteforce_codes(xv[r], s[r, 0])


def test_representable_blocks_round_trip():
    rng = np.random.default_rng(6)
    for _ in range(50):
        k = int(rng.integers(-100, 100))
        mags = formats.E4M3_POS[rng.integers(0, 127, 32)]
        mags[0] = formats.E4M3_POS[int(rng.integers(0x78, 0x7F))]          # max in [256, 448]
        signs = np.where(rng.random(32) < 0.5, -1.0, 1.0)
        v = np.ldexp(mags * signs, k)
        bits = f32_to_bf16_bits(v.astype(np.float32))[None, :]
        assert np.array_equal(formats.bf16_to_f64(bits[0]), v)             # bf16 holds them exactly
        c, s = quant.quantize_mx8(bits)
        assert int(s[0, 0]) == 127 + k
        np.testing.assert_array_equal(quant.dequantize_mx8(c, s)[0], v)


def test_quantization_error_bound():
    bits = _blocks(np.random.default_rng(7), 2000)
    c, s = quant.quantize_mx8(bits)
    xv = formats.bf16_to_f64(bits)
    deq = quant.dequantize_mx8(c, s)
    scale = np.repeat(formats.e8m0_decode(s), 32, axis=1)
    v = np.abs(xv) / scale
    err = np.abs(deq - xv)
    normal = (v >= 2.0 ** -6) & (v <= 448)
    assert np.all(err[normal] <= np.abs(xv[normal]) * 2.0 ** -4)
    sub = v < 2.0 ** -6
    assert np.all(err[sub] <= 2.0 ** -10 * scale[sub])
    sat = v > 448
    np.testing.assert_array_equal(np.abs(deq[sat]), 448.0 * scale[sat])
    assert np.all(np.signbit(deq) == np.signbit(xv))


def test_gemm_matches_exact_rational_sum():
    rng = np.random.default_rng(8)
    M, N, K = 3, 4, 96
    x = rng.standard_normal((M, K)).astype(np.float32) * (2.0 ** rng.integers(-6, 6, (M, K))).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32) * 0.05
    a = quant.quantize_mx8(f32_to_bf16_bits(x))
    b = quant.quantize_mx8(f32_to_bf16_bits(w))
    acc = gemm.gemm_mx8(a[0], a[1], b[0], b[1])
    ad, bd = formats.e4m3_decode(a[0]), formats.e4m3_decode(b[0])
    for m in range(M):
        for n in range(N):
            exact, mag = Fraction(0), Fraction(0)
            for k in range(K):
                t = (Fraction(float(ad[m, k])) * 2 ** (int(a[1][m, k // 32]) - 127)
                     * Fraction(float(bd[n, k])) * 2 ** (int(b[1][n, k // 32]) - 127))
                exact += t
                mag += abs(t)
            assert abs(Fraction(float(acc[m, n])) - exact) <= mag * Fraction(1, 2 ** 40)
    rows = gemm.gemm_mx8(a[0], a[1], b[0], b[1], rows=[2, 0])
    np.testing.assert_array_equal(rows, acc[[2, 0]])


def test_gemm_with_unit_scales_is_the_plain_e4m3_product():
    rng = np.random.default_rng(9)
    ac = rng.integers(0, 256, (5, 64), dtype=np.uint8)
    wc = rng.integers(0, 256, (7, 64), dtype=np.uint8)
    ac[(ac & 0x7F) == 0x7F] = 0                            # no NaN codes
    wc[(wc & 0x7F) == 0x7F] = 0
    ones_a = np.full((5, 2), 127, np.uint8)
    ones_w = np.full((7, 2), 127, np.uint8)
    got = gemm.gemm_mx8(ac, ones_a, wc, ones_w)
    ref = gemm.gemm_fp8(ac, np.ones(5, np.float32), wc, np.ones(7, np.float32))
    np.testing.assert_array_equal(got, ref)
