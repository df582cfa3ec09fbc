"""Pins of the packed-blob decoder: a writer built here from the documented
layout (explicit loops, one element at a time) and the decoder must invert each
other, and the gated-SiLU interleave must place each gate row and its up row in
the same lane of two adjacent 32-row groups."""
import numpy as np
import pytest

from oracle import packed


def _write_blob(codes, scales, fmt, epi, N, K):
    Np = packed.padded_rows(N)
    perm = packed.row_perm(epi, N, Np)
    if fmt == packed.FMT_FP4:
        cbytes, sbytes = Np * K // 2, Np * K // 32
    elif fmt == packed.FMT_MX8:
        cbytes, sbytes = Np * K, Np * K // 32
    elif fmt == packed.FMT_NV4:
        cbytes, sbytes = Np * K // 2, Np * K // 16
    else:
        cbytes, sbytes = Np * K, Np * 4
    blob = np.zeros(packed.HEADER + cbytes + sbytes, dtype=np.uint8)
    hdr = np.zeros(64, dtype=np.uint8)
    hdr[:28] = np.array([packed.MAGIC, 2, fmt, epi, N, K, Np], dtype=np.uint32).view(np.uint8)
    hdr[32:56] = np.array([256, 256 + cbytes, blob.size], dtype=np.uint64).view(np.uint8)
    blob[:64] = hdr
    for p in range(Np):
        n = perm[p]
        if n < 0:
            continue
        g, lane_lo = p // 32, p % 32
        if fmt in (packed.FMT_FP4, packed.FMT_NV4):
            for k in range(0, K, 2):
                c, within = k // 64, k % 64
                L = lane_lo + 32 * (within // 32)
                b = (within % 32) // 2
                blob[256 + (g * (K // 64) + c) * 1024 + 16 * L + b] = codes[n, k // 2]
            if fmt == packed.FMT_NV4:
                for blk in range(K // 16):
                    s, r = blk // 8, blk % 8                 # r = 4j + 2 * half + b
                    j, half, bb = r // 4, (r // 2) % 2, r % 2
                    L = lane_lo + 32 * half
                    blob[256 + cbytes + (s * (Np // 32) + g) * 256 + 4 * L + 2 * j + bb] = scales[n, blk]
                continue
            for blk in range(K // 32):
                s, r = blk // 4, blk % 4
                j, half = r // 2, r % 2
                L = lane_lo + 32 * half
                blob[256 + cbytes + (s * (Np // 32) + g) * 128 + 2 * L + j] = scales[n, blk]
        else:
            for k in range(K):
                c, within = k // 64, k % 64
                L = lane_lo + 32 * ((within % 32) // 16)
                byte = 16 * (within // 32) + within % 16
                blob[256 + (g * (K // 64) + c) * 2048 + 32 * L + byte] = codes[n, k]
            if fmt == packed.FMT_MX8:
                for blk in range(K // 32):
                    s, r = blk // 4, blk % 4
                    L = lane_lo + 32 * (r % 2)
                    blob[256 + cbytes + (s * (Np // 32) + g) * 128 + 2 * L + r // 2] = scales[n, blk]
            else:
                blob[256 + cbytes + 4 * p:256 + cbytes + 4 * p + 4] = np.array([scales[n]], np.float32).view(np.uint8)
    return blob


@pytest.mark.parametrize("fmt,epi,N,K", [(1, 0, 64, 256), (1, 1, 128, 512), (1, 2, 300 - 300 % 32 + 32, 256),
                                         (2, 0, 96, 256), (2, 1, 128, 256), (3, 0, 96, 256), (3, 1, 128, 512),
                                         (3, 2, 64, 384), (4, 0, 64, 256), (4, 1, 128, 512)])
def test_writer_and_decoder_invert(fmt, epi, N, K):
    rng = np.random.default_rng(N + K + fmt)
    if fmt == 1:
        codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        scales = rng.integers(100, 150, (N, K // 32), dtype=np.uint8)
    elif fmt == 3:
        codes = rng.integers(0, 256, (N, K), dtype=np.uint8)
        scales = rng.integers(100, 150, (N, K // 32), dtype=np.uint8)
    elif fmt == 4:
        codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        scales = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)
    else:
        codes = rng.integers(0, 256, (N, K), dtype=np.uint8)
        scales = rng.uniform(0.01, 1, N).astype(np.float32)
    blob = _write_blob(codes, scales, fmt, epi, N, K)
    hdr = packed.read_header(blob)
    assert hdr["magic"] == packed.MAGIC and hdr["N"] == N and hdr["K"] == K and hdr["Np"] == packed.padded_rows(N)
    c2, s2, pad = packed.decode(blob, fmt, epi, N, K)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scales)
    assert not pad["codes"].any()


def test_gated_interleave_pairs_share_a_lane():
    N = 512
    Np = packed.padded_rows(N)
    perm = packed.row_perm(packed.EPI_GATED_SILU, N, Np)
    for p in range(0, N, 64):
        for i in range(32):
            gate, up = perm[p + i], perm[p + 32 + i]
            assert up == gate + N // 2
            assert gate == p // 2 + i
    assert sorted(perm[:N]) == list(range(N))
