"""Helpers shared by the GPU parity tests (device transfer, tolerance check)."""
from __future__ import annotations

import numpy as np

from workloads import bf16_bits_to_f32

# Per-element reading of the tolerance for bf16 outputs: the output must lie within
# 8e-3 x row-RMS of the float64 oracle plus half a bf16 ulp of the oracle value
# (the rounding every bf16 store makes).  Without the half-ulp term no bf16 output
# can meet the bound on rows whose largest elements exceed ~4x their RMS.
RMS_TOL = 8e-3


def to_dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def to_host_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def act_codes_to_rowmajor(codes: np.ndarray, M: int, K: int, fmt: int) -> np.ndarray:
    """dit_quantize_act's K-panel-major codes -> row-major (FP4 [M, K/2], FP8 [M, K]).

    Follows the layout include/ditq.h documents: FP4 panels of 128 K elements
    (64 bytes per token), FP8 panels of 64 elements (64 bytes per token).
    """
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    panels = (K // 128) if fmt == 1 else (K // 64)
    return c.reshape(panels, M, 64).transpose(1, 0, 2).reshape(M, panels * 64)


def act_scales_to_rowmajor(scales: np.ndarray, M: int, K: int) -> np.ndarray:
    """FP4 scale bytes, [K/128][M][4] -> [M, K/32] (block b of token m)."""
    s = np.asarray(scales, dtype=np.uint8).reshape(-1)
    return s.reshape(K // 128, M, 4).transpose(1, 0, 2).reshape(M, K // 32)


def half_ulp_bf16(y: np.ndarray) -> np.ndarray:
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def compare_bf16(gpu_bits: np.ndarray, y: np.ndarray, label: str = "") -> dict:
    """Check a bf16 GPU output against the float64 oracle; raise with details on failure."""
    g = bf16_bits_to_f32(gpu_bits).astype(np.float64)
    assert g.shape == y.shape, (g.shape, y.shape)
    assert np.all(np.isfinite(g)), f"{label}: non-finite output"
    rms = np.sqrt(np.mean(y * y, axis=1))
    err = np.abs(g - y)
    bound = RMS_TOL * rms[:, None] + half_ulp_bf16(y)
    bad = err > bound
    literal = float((err.max(axis=1) / np.where(rms > 0, rms, 1.0)).max())
    rep = {"literal_max_err_over_rowrms": literal, "bad": int(bad.sum()), "n": int(err.size),
           "max_err_over_bound": float((err / np.maximum(bound, 1e-300)).max())}
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {rep['bad']} of {rep['n']} elements out of tolerance; first at "
                             f"[{i},{j}] gpu={g[i, j]!r} oracle={y[i, j]!r} rowrms={rms[i]!r}; {rep}")
    return rep


def nv4_act_scales(scales: np.ndarray, M: int, K: int):
    """NVFP4 activation scales buffer -> (E4M3 block scale codes [M, K/16], fp32 tensor scale)."""
    s = np.asarray(scales, dtype=np.uint8).reshape(-1)
    blocks = s[:M * K // 16].reshape(K // 128, M, 8).transpose(1, 0, 2).reshape(M, K // 16)
    st = s[M * K // 16 + 4:M * K // 16 + 8].copy().view(np.float32)[0]
    return blocks, st
