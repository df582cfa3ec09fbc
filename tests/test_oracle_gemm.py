"""Pins of the oracle's decode-multiply GEMM.

* exact-rational brute force (Python loops over fractions.Fraction) on tiny
  problems equals the float64 oracle exactly, FP4 and FP8 (catches a transposed
  operand, a wrong scale index or a dropped term);
* closed-form special cases: all-ones, a one-hot weight that copies a column of
  the dequantized activations, a single non-zero block.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats, gemm, quant
from workloads import f32_to_bf16_bits


def _frac_fp4(packed, scales, r, k):
    byte = packed[r, k // 2]
    code = (byte & 0xF) if k % 2 == 0 else (byte >> 4)
    mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)][code & 7]
    if code & 8:
        mag = -mag
    return mag * Fraction(2) ** (int(scales[r, k // 32]) - 127)


def _rand_bits(rng, shape, spread=4):
    x = rng.standard_normal(shape).astype(np.float32) * (2.0 ** rng.integers(-spread, spread, shape)).astype(np.float32)
    return f32_to_bf16_bits(x)


@pytest.mark.parametrize("M,N,K,seed", [(4, 8, 64, 0), (3, 5, 96, 1), (2, 33, 128, 2)])
def test_fp4_gemm_equals_rational_brute_force(M, N, K, seed):
    rng = np.random.default_rng(seed)
    ac, as_ = quant.quantize_fp4(_rand_bits(rng, (M, K)))
    wc, ws = quant.quantize_fp4(_rand_bits(rng, (N, K)))
    acc = gemm.gemm_fp4(ac, as_, wc, ws)
    for m in range(M):
        for n in range(N):
            exact = sum((_frac_fp4(ac, as_, m, k) * _frac_fp4(wc, ws, n, k) for k in range(K)), Fraction(0))
            assert Fraction(float(acc[m, n])) == exact, (m, n)


def test_fp4_gemm_tiny_workload_exact():
    from workloads import make_inputs
    d = make_inputs("tiny_gated_silu", seed=0)
    ac, as_ = quant.quantize_fp4(d["x"])
    wc, ws = quant.quantize_fp4(d["w"])
    acc = gemm.gemm_fp4(ac, as_, wc, ws)
    rng = np.random.default_rng(5)
    for _ in range(40):
        m, n = int(rng.integers(64)), int(rng.integers(512))
        exact = sum((_frac_fp4(ac, as_, m, k) * _frac_fp4(wc, ws, n, k) for k in range(256)), Fraction(0))
        assert Fraction(float(acc[m, n])) == exact


def test_fp8_gemm_equals_rational_brute_force():
    rng = np.random.default_rng(7)
    M, N, K = 3, 6, 64
    ac, as_ = quant.quantize_fp8(_rand_bits(rng, (M, K)))
    wc, ws = quant.quantize_fp8(_rand_bits(rng, (N, K)))
    acc = gemm.gemm_fp8(ac, as_, wc, ws)
    da, dw = formats.e4m3_decode(ac), formats.e4m3_decode(wc)
    for m in range(M):
        for n in range(N):
            exact = sum((Fraction(float(da[m, k])) * Fraction(float(dw[n, k])) for k in range(K)), Fraction(0))
            exact *= Fraction(float(as_[m])) * Fraction(float(ws[n]))
            assert abs(Fraction(float(acc[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 51)


def test_all_ones_gives_K():
    K = 256
    codes = np.full((2, K // 2), 0x22, dtype=np.uint8)        # 1.0 in both nibbles
    scales = np.full((2, K // 32), 127, dtype=np.uint8)
    acc = gemm.gemm_fp4(codes, scales, codes, scales)
    assert np.all(acc == K)


def test_one_hot_weight_copies_activation_column():
    rng = np.random.default_rng(9)
    K = 128
    ac, as_ = quant.quantize_fp4(_rand_bits(rng, (5, K)))
    wc = np.zeros((3, K // 2), dtype=np.uint8)
    ws = np.full((3, K // 32), 127, dtype=np.uint8)
    cols = [3, 64, 127]
    for n, k in enumerate(cols):
        wc[n, k // 2] = 0x2 if k % 2 == 0 else 0x20
    acc = gemm.gemm_fp4(ac, as_, wc, ws)
    np.testing.assert_array_equal(acc, quant.dequantize_fp4(ac, as_)[:, cols])


def test_single_block_is_a_scaled_dot_product():
    rng = np.random.default_rng(11)
    K = 256
    ac, as_ = quant.quantize_fp4(_rand_bits(rng, (1, K)))
    wc, ws = quant.quantize_fp4(_rand_bits(rng, (1, K)))
    wc[:, :] = 0
    wc[0, 16 * 3:16 * 4] = rng.integers(0, 256, 16, dtype=np.uint8)      # block 3 only
    acc = gemm.gemm_fp4(ac, as_, wc, ws)[0, 0]
    a = formats.e2m1_decode(quant.unpack_fp4_codes(ac)[0, 96:128])
    w = formats.e2m1_decode(quant.unpack_fp4_codes(wc)[0, 96:128])
    ref = float(np.dot(a, w)) * 2.0 ** (int(as_[0, 3]) - 127) * 2.0 ** (int(ws[0, 3]) - 127)
    assert acc == ref


def test_exactness_guard_rejects_extreme_exponent_spread():
    K = 64
    s = np.array([[1, 254]], dtype=np.uint8)
    assert not gemm.fp4_sum_is_exact(s, s, K)
    with pytest.raises(ArithmeticError):
        gemm.gemm_fp4(np.zeros((1, 32), np.uint8), s, np.zeros((1, 32), np.uint8), s)
