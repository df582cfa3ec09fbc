"""Index model of the gated-residual epilogue's reads (CPU).

The fused epilogue out = residual + gate[m / rows_per_gate] * C reads the residual
and the gate table of every column its result tile covers.  The tiles cover the
padded width Np = ceil(N / 256) * 256 and whole 32-token slices past M, so the
reads must be clipped: rows past M read row M - 1, and a 32-column result tile that
starts at or past N reads nothing (4-bit formats) or the last 32 columns (8-bit).  This test replays the kernel's address arithmetic (2 x 2 wave grid,
128 features x 32*TM tokens per wave, lane l: token l % 32, runs 8g + 4(l / 32) of
each 32-column result tile) for the fuzz shapes and the full-size workload, and
checks that every element read lies inside the documented extents:
residual[(M - 1) * ldr + N] (bf16 [M][ldr]) and gate[ceil(M / rows_per_gate) * N].
Without the column clip the model reads past both extents whenever N % 256 != 0,
which the last test shows.
"""
import numpy as np
import pytest

from tests.test_gpu_fuzz import _cases


def tm_for(fmt: str, M: int, N: int, cus: int = 256) -> int:
    """Token tiles per wave the launcher picks for the gated residual (2 x 2 grid)."""
    if fmt != "fp4":
        return 3
    tn = (N + 255) // 256
    r3 = ((M + 191) // 192 * tn + cus - 1) // cus
    r4 = ((M + 255) // 256 * tn + cus - 1) // cus
    return 3 if r3 * 20 < r4 * 27 else 4


def reads(M, N, ldr, rpg, TM, clip_columns=True, fmt="fp4"):
    """Element indices of every residual and gate read the epilogue makes.  A result
    tile that starts at or past N: the 4-bit formats skip its reads, the 8-bit ones
    read the last 32 columns instead."""
    WN, WM = 128, 32 * TM
    BN, BM = 2 * WN, 2 * WM
    Np = (N + 255) // 256 * 256
    tiles_m, tiles_n = (M + BM - 1) // BM, Np // BN
    m0 = np.arange(tiles_m)[:, None, None, None, None, None, None] * BM
    n0 = np.arange(tiles_n)[None, :, None, None, None, None, None] * BN
    wn = np.arange(2)[None, None, :, None, None, None, None]
    wm = np.arange(2)[None, None, None, :, None, None, None]
    lane = np.arange(64)[None, None, None, None, :, None, None]
    tm = np.arange(TM)[None, None, None, None, None, :, None]
    tn = np.arange(4)[None, None, None, None, None, None, :]
    row = m0 + wm * WM + 32 * tm + (lane & 31)
    rr = np.where(row < M, row, M - 1)
    tile_col = n0 + wn * WN + 32 * tn                # first column of the 32-column result tile
    skip = fmt in ("fp4", "nv4") or not clip_columns
    col = (tile_col if skip else np.minimum(tile_col, N - 32)) + 4 * (lane >> 5)
    res, gat = [], []
    for g in range(4):
        c = col + 8 * g
        # the kernel reads a result tile only when it starts before N (a test uniform
        # over the wave; N % 64 == 0, so a tile is wholly in or out)
        take = np.broadcast_to(tile_col < N, np.broadcast(rr, c).shape) if clip_columns and skip else \
            np.ones(np.broadcast(rr, c).shape, dtype=bool)
        r_b = np.broadcast_to(rr, take.shape)[take].astype(np.int64)
        c_b = np.broadcast_to(c, take.shape)[take].astype(np.int64)
        for i in range(4):
            res.append(r_b * ldr + c_b + i)
            gat.append((r_b // rpg) * N + c_b + i)
    return np.concatenate(res), np.concatenate(gat)


def check(M, N, ldr, rpg, TM, fmt):
    res, gat = reads(M, N, ldr, rpg, TM, fmt=fmt)
    assert res.min() >= 0 and res.max() < (M - 1) * ldr + N, (M, N, ldr, rpg, TM, int(res.max()))
    assert gat.min() >= 0 and gat.max() < (M + rpg - 1) // rpg * N, (M, N, ldr, rpg, TM, int(gat.max()))
    # every output element's residual and gate value is read
    assert np.unique(res).size == M * N
    return res, gat


GR_CASES = [c for c in _cases() if c[2] == "gate_residual"]


@pytest.mark.parametrize("case", GR_CASES, ids=[f"fuzz{c[0]}" for c in GR_CASES])
def test_fuzz_shapes_read_inside_extents(case):
    i, fmt, _, M, N, K, _, rpg, pad = case
    # the fuzz runs the residual with ldr = N (exact rows) and the output with ldo = N + pad
    check(M, N, N, rpg, tm_for(fmt, M, N), fmt)


@pytest.mark.parametrize("fmt,M,N,ldr,rpg", [("fp4", 9216, 3072, 3072, 4608), ("fp4", 300, 576, 576, 7),
                                            ("fp8", 257, 320, 328, 129), ("mx8", 1, 64, 64, 1),
                                            ("nv4", 193, 1600, 1600, 193)])
def test_chosen_shapes_read_inside_extents(fmt, M, N, ldr, rpg):
    check(M, N, ldr, rpg, tm_for(fmt, M, N), fmt)


def test_model_detects_reads_past_the_extents_without_the_column_clip():
    M, N, rpg = 300, 576, 7                     # N % 256 = 64: the last tile is mostly padding
    res, gat = reads(M, N, N, rpg, tm_for("fp4", M, N), clip_columns=False)
    assert res.max() >= (M - 1) * N + N and gat.max() >= (M + rpg - 1) // rpg * N
