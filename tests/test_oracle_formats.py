"""Pins of the oracle's format decoders: closed forms and two independent decoders."""
import numpy as np

from oracle import formats


def test_e2m1_table_and_bitfield_agree_on_all_16_codes():
    codes = np.arange(16)
    a = formats.e2m1_decode(codes)
    b = formats.e2m1_decode_bitfield(codes)
    np.testing.assert_array_equal(np.signbit(a), np.signbit(b))
    np.testing.assert_array_equal(a, b)
    # the magnitudes the E2M1 definition fixes: subnormal 0.5, then 1, 1.5, 2, 3, 4, 6
    np.testing.assert_array_equal(a[:8], [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    np.testing.assert_array_equal(a[8:], -a[:8])


def test_e8m0():
    v = formats.e8m0_decode(np.array([0, 1, 126, 127, 128, 254, 255]))
    np.testing.assert_array_equal(v[:6], [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 2.0 ** 127])
    assert np.isnan(v[6])


def test_e4m3_bitfield_and_table_agree_on_all_256_codes():
    codes = np.arange(256)
    a = formats.e4m3_decode(codes)
    b = formats.e4m3_decode_table(codes)
    nan = np.isnan(a)
    np.testing.assert_array_equal(nan, np.isnan(b))
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(a[~nan], b[~nan])
    assert a[0x38] == 1.0 and a[0x7E] == 448.0 and a[0x01] == 2.0 ** -9 and a[0x08] == 2.0 ** -6
    assert a[0x77] == 240.0 and a[0x78] == 256.0 and a[0xC5] == -3.25
    # strictly increasing over the finite non-negative codes
    assert np.all(np.diff(a[:0x7F]) > 0)


def test_bf16_decoders_agree_on_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    a = formats.bf16_to_f64(bits)
    b = formats.bf16_to_f64_bitfield(bits)
    fin = np.isfinite(a)
    np.testing.assert_array_equal(fin, np.isfinite(b))
    np.testing.assert_array_equal(np.isnan(a), np.isnan(b))
    np.testing.assert_array_equal(a[fin], b[fin])
    np.testing.assert_array_equal(np.signbit(a[fin]), np.signbit(b[fin]))
    assert formats.bf16_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert formats.bf16_to_f64(np.array([0x0001], np.uint16))[0] == 2.0 ** -133
