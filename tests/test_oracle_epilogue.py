"""Pins of the oracle's epilogues: closed forms and invariants.

gated-SiLU (page "How fal made Ideogram V4 6x faster", paragraph 4):
  SiLU(0) = 0, SiLU(x) - SiLU(-x) = x, finite for very negative x, and the first
  half of the columns is the gate (a swapped half fails).
per-head QK-RMSNorm (same page, paragraph 3):
  a constant head c gives c / sqrt(c^2 + eps) * gamma; mean((y/gamma)^2) equals
  ms / (ms + eps); scale invariance up to eps; V untouched; Q heads use gamma_q and
  K heads gamma_k.
"""
import math

import numpy as np
import pytest

from oracle import epilogue


def test_silu_closed_forms():
    x = np.linspace(-30, 30, 601)
    s = epilogue.silu(x)
    assert epilogue.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s - epilogue.silu(-x), x, rtol=0, atol=1e-12)
    assert epilogue.silu(np.array([1.0]))[0] == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-15)
    big = epilogue.silu(np.array([-1e4, 1e4]))
    assert big[0] == 0.0 and big[1] == 1e4


def test_gated_silu_uses_first_half_as_gate():
    rng = np.random.default_rng(0)
    g = rng.standard_normal((5, 8))
    acc = np.concatenate([g, np.ones((5, 8))], axis=1)
    np.testing.assert_array_equal(epilogue.gated_silu(acc), epilogue.silu(g))
    u = rng.standard_normal((5, 8))
    acc = np.concatenate([g, u], axis=1)
    np.testing.assert_allclose(epilogue.gated_silu(acc), g / (1 + np.exp(-g)) * u, rtol=1e-15)


@pytest.mark.parametrize("D", [128, 256])
def test_rmsnorm_constant_head(D):
    H, eps = 2, 1e-6
    gq = np.linspace(0.5, 1.5, D)
    gk = np.linspace(1.5, 0.5, D)
    acc = np.zeros((3, 3 * H * D))
    c = np.array([0.001, 1.0, -7.0])
    acc[:, :] = c[:, None]
    y = epilogue.qk_rmsnorm(acc, H, D, gq, gk, eps)
    f = c / np.sqrt(c * c + eps)
    np.testing.assert_allclose(y[:, :D], f[:, None] * gq, rtol=1e-14)
    np.testing.assert_allclose(y[:, H * D:H * D + D], f[:, None] * gk, rtol=1e-14)
    np.testing.assert_array_equal(y[:, 2 * H * D:], acc[:, 2 * H * D:])


@pytest.mark.parametrize("D", [128, 256])
def test_rmsnorm_invariants(D):
    rng = np.random.default_rng(D)
    H, eps = 3, 1e-6
    gq = rng.uniform(0.5, 1.5, D)
    gk = rng.uniform(0.5, 1.5, D)
    acc = rng.standard_normal((4, 3 * H * D)) * rng.uniform(0.01, 50, (4, 1))
    y = epilogue.qk_rmsnorm(acc, H, D, gq, gk, eps)
    for part, g in ((0, gq), (1, gk)):
        for h in range(H):
            cols = slice(part * H * D + h * D, part * H * D + (h + 1) * D)
            x = acc[:, cols]
            ms = np.mean(x * x, axis=1)
            np.testing.assert_allclose(np.mean((y[:, cols] / g) ** 2, axis=1), ms / (ms + eps), rtol=1e-12)
    y2 = epilogue.qk_rmsnorm(acc * 3.0, H, D, gq, gk, eps)
    np.testing.assert_allclose(y2[:, :2 * H * D], y[:, :2 * H * D], rtol=1e-5)
    np.testing.assert_array_equal(y[:, 2 * H * D:], acc[:, 2 * H * D:])


def test_rmsnorm_head_is_local_and_per_head():
    D, H = 128, 2
    acc = np.ones((1, 3 * H * D))
    acc[0, D:2 * D] = 100.0                    # second Q head much larger: must not affect the first
    y = epilogue.qk_rmsnorm(acc, H, D, np.ones(D), np.ones(D), 0.0)
    np.testing.assert_allclose(y[0, :2 * D], 1.0, rtol=1e-15)


def test_gelu_tanh_closed_forms_and_library():
    import torch
    x = np.concatenate([np.linspace(-12, 12, 2401), [-1e4, -50.0, 50.0, 1e4, 1e30, -1e30]])
    g = epilogue.gelu_tanh(x)
    assert epilogue.gelu_tanh(np.array([0.0]))[0] == 0.0
    # x * Phi-like form: g(x) - g(-x) = x for the tanh form too (tanh is odd)
    np.testing.assert_allclose(g - epilogue.gelu_tanh(-x), x, rtol=1e-15, atol=1e-12)
    # torch's tanh-approximated GELU in float64 on the CPU
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    # (1 + tanh u) cancels for very negative x in both, so the tails agree only to ~1e-15 absolute
    np.testing.assert_allclose(g, ref, rtol=1e-14, atol=1e-15)
    # within the tanh approximation's known distance of the exact GELU x * Phi(x)
    from scipy.special import erf
    exact = 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))
    small = np.abs(x) < 20
    assert np.max(np.abs(g[small] - exact[small])) < 1e-3
    assert g[-1] == 0.0 and g[-3] == 1e4 and g[-4] == 50.0


def test_gate_residual_against_elementwise_loops():
    rng = np.random.default_rng(3)
    from workloads import f32_to_bf16_bits
    M, N, rpg = 7, 5, 3
    acc = rng.standard_normal((M, N))
    res = f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    gate = rng.standard_normal(((M + rpg - 1) // rpg, N)).astype(np.float32)
    y = epilogue.gate_residual(acc, res, gate, rpg)
    rv = (res.astype(np.uint32) << 16).view(np.float32)
    for m in range(M):
        for n in range(N):
            assert y[m, n] == float(rv[m, n]) + float(gate[m // rpg, n]) * acc[m, n]
    rows = np.array([6, 0, 4])
    np.testing.assert_array_equal(epilogue.gate_residual(acc[rows], res, gate, rpg, row_ids=rows), y[rows])
    np.testing.assert_array_equal(epilogue.gate_residual(acc, res, np.zeros_like(gate), rpg), rv.astype(np.float64))
    np.testing.assert_array_equal(epilogue.gate_residual(acc, np.zeros_like(res), np.ones_like(gate), rpg), acc)
