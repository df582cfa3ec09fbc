"""Pins of the oracle's NVFP4 quantizer (E2M1 elements, E4M3 scale per 16 K
elements, fp32 tensor scale) and of its decode-multiply GEMM.

* hand-derived worked tensors (tests/golden/nv4_worked_examples.txt);
* the block holding the tensor maximum gets the largest scale code (448) and its
  maximum the largest element code (6), for any tensor;
* every block scale is the E4M3 value nearest to fl32(amax_b / fl32(6 s_t)) (a
  search over all E4M3 values);
* every element code, recomputed in exact rational arithmetic (the two fp32
  roundings of the definition done on exact rationals), then the nearest E2M1
  grid point by search;
* exact round trips of representable tensors, the all-zero tensor;
* the GEMM against exact rational sums.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats, gemm, quant
from tests.conftest import read_golden
from tests.test_oracle_quant_fp8 import _rn32
from workloads import f32_to_bf16_bits


@pytest.mark.parametrize("row", read_golden("nv4_worked_examples.txt"), ids=lambda r: r[1][:20])
def test_tensor_examples(row):
    _, blocks, st, scales, codes = row
    blocks = [b.split() for b in blocks.split(";")]
    bits = np.zeros((1, 16 * len(blocks)), dtype=np.uint16)
    for i, b in enumerate(blocks):
        bits[0, 16 * i:16 * i + len(b)] = [int(t, 16) for t in b]
    c, s, s_t = quant.quantize_nv4(bits)
    assert float(s_t) == float(st)
    assert [int(v) for v in s[0]] == [int(t, 16) for t in scales.split()]
    u = quant.unpack_fp4_codes(c)[0]
    for i, want in enumerate(codes.split(";")):
        want = [int(t, 16) for t in want.split()]
        assert [int(v) for v in u[16 * i:16 * i + len(want)]] == want
        assert not (u[16 * i + len(want):16 * i + 16] & 7).any()


def _tensor(rng, R, K):
    x = rng.standard_normal((R, K)).astype(np.float32) * (2.0 ** rng.integers(-8, 8, (R, 1))).astype(np.float32)
    x[:, rng.integers(0, K, max(1, K // 50))] *= 20.0
    x[rng.random((R, K)) < 0.03] = 0.0
    x[rng.random((R, K)) < 0.01] *= -0.0
    return f32_to_bf16_bits(x)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tensor_maximum_block(seed):
    bits = _tensor(np.random.default_rng(seed), 8, 256)
    c, s, s_t = quant.quantize_nv4(bits)
    x = formats.bf16_to_f64(bits)
    r, k = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert s[r, k // 16] == 0x7E
    assert quant.unpack_fp4_codes(c)[r, k] & 7 == 7
    assert np.all(formats.e4m3_decode(s) <= 448)


def test_block_scales_are_nearest_e4m3():
    bits = _tensor(np.random.default_rng(5), 16, 512)
    c, s, s_t = quant.quantize_nv4(bits)
    x = formats.bf16_to_f64(bits)
    six_st = Fraction(float(_rn32(Fraction(6) * Fraction(float(s_t)))))
    grid = formats.E4M3_POS
    for r in range(16):
        for b in range(512 // 16):
            amax = Fraction(float(np.abs(x[r, 16 * b:16 * b + 16]).max()))
            d = min(float(_rn32(amax / six_st)), 448.0)
            dist = np.abs(grid - d)
            best = np.flatnonzero(dist == dist.min())
            want = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
            assert s[r, b] == want, (r, b, d)


def test_element_codes_by_exact_arithmetic():
    bits = _tensor(np.random.default_rng(6), 4, 128)
    c, s, s_t = quant.quantize_nv4(bits)
    u = quant.unpack_fp4_codes(c)
    x = formats.bf16_to_f64(bits)
    grid = formats.E2M1_GRID
    for r in range(4):
        for k in range(128):
            sb = float(formats.e4m3_decode(s[r, k // 16]))
            sign = 8 if np.signbit(x[r, k]) else 0
            if sb == 0:
                assert u[r, k] == sign
                continue
            denom = _rn32(Fraction(sb) * Fraction(float(s_t)))
            y = min(abs(float(_rn32(Fraction(float(x[r, k])) / Fraction(float(denom))))), 6.0)
            dist = np.abs(grid - y)
            best = np.flatnonzero(dist == dist.min())
            want = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
            assert u[r, k] == want | sign, (r, k)


def test_representable_tensors_round_trip():
    rng = np.random.default_rng(7)
    for _ in range(20):
        k = int(rng.integers(-20, 20))
        R, K = 3, 64
        s_blocks = formats.E4M3_POS[rng.integers(0x20, 0x7F, (R, K // 16))]
        s_blocks[0, 0] = 448.0
        q = formats.E2M1_GRID[rng.integers(0, 8, (R, K))] * np.where(rng.random((R, K)) < 0.5, -1, 1)
        for r in range(R):
            for b in range(K // 16):
                q[r, 16 * b] = 6.0                                     # each block reaches 6 * its scale
        v = q * np.repeat(s_blocks, 16, axis=1) * 2.0 ** k
        bits = f32_to_bf16_bits(v.astype(np.float32))
        assert np.array_equal(formats.bf16_to_f64(bits), v)
        c, s, s_t = quant.quantize_nv4(bits)
        assert float(s_t) == 2.0 ** k
        np.testing.assert_array_equal(formats.e4m3_decode(s), s_blocks)
        np.testing.assert_array_equal(quant.dequantize_nv4(c, s, s_t), v)


def test_zero_tensor():
    bits = np.zeros((2, 32), np.uint16)
    bits[1, 5] = 0x8000
    c, s, s_t = quant.quantize_nv4(bits)
    assert float(s_t) == 1.0 and not s.any()
    u = quant.unpack_fp4_codes(c)
    assert u[1, 5] == 8 and int(u.sum()) == 8


def test_gemm_matches_exact_rational_sum():
    rng = np.random.default_rng(8)
    M, N, K = 3, 4, 64
    a = quant.quantize_nv4(_tensor(rng, M, K))
    w = quant.quantize_nv4(f32_to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * 0.05))
    acc = gemm.gemm_nv4(a[0], a[1], a[2], w[0], w[1], w[2])
    ad = formats.e2m1_decode(quant.unpack_fp4_codes(a[0]))
    wd = formats.e2m1_decode(quant.unpack_fp4_codes(w[0]))
    sa, sw = formats.e4m3_decode(a[1]), formats.e4m3_decode(w[1])
    st = Fraction(float(a[2])) * Fraction(float(w[2]))
    for m in range(M):
        for n in range(N):
            exact, mag = Fraction(0), Fraction(0)
            for k in range(K):
                t = Fraction(float(ad[m, k])) * Fraction(float(sa[m, k // 16])) * \
                    Fraction(float(wd[n, k])) * Fraction(float(sw[n, k // 16])) * st
                exact += t
                mag += abs(t)
            assert abs(Fraction(float(acc[m, n])) - exact) <= mag * Fraction(1, 2 ** 40)
