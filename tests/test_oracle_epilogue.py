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
