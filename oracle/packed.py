"""Decoder of the packed weight blob, written from its documented layout.

Test infrastructure (see the package docstring).  It reads the byte layout that
``include/ditq.h`` documents for ``dit_pack_weights`` and returns the logical
codes and scales, so the packer can be compared bit-exactly with the oracle
quantizer applied to the same weights.  It shares no code with the packer.

Layout (all offsets in bytes, little-endian):

* header, 256 bytes: u32 magic 0x51544944 ("DITQ"), u32 layout version (2),
  u32 fmt, u32 epi, u32 N, u32 K, u32 Np (N rounded up to 256), u32 0,
  u64 codes offset (256), u64 scales offset, u64 total bytes, zeros.
* packed row p (0 <= p < Np) holds logical weight row perm(p):
  identity / QK-RMSNorm: perm(p) = p; gated-SiLU: with P = p // 64, i = p % 64,
  perm(p) = 32P + i for i < 32 (gate) and N/2 + 32P + (i - 32) otherwise (up),
  so each gate row and its up row sit in the same lane of two adjacent 32-row
  groups.  Rows p >= N are zero padding.
* FP4 codes: 1024-byte fragments, fragment (g, c) for row group g < Np/32 and
  K chunk c < K/64 at codes_offset + (g * K/64 + c) * 1024; byte 16*L + b
  (lane L < 64, b < 16) holds the codes of packed row 32g + L%32 at
  k = 64c + 32(L//32) + 2b (low nibble) and k + 1 (high nibble).
* FP4 scales: 128-byte records, record (s, g) for K step s < K/128 and row
  group g < Np/32 at scales_offset + (s * Np/32 + g) * 128; byte 2*L + j holds the
  E8M0 scale of packed row 32g + L%32 for the 32-element K block 4s + 2j + L//32.
* FP8 codes: 2048-byte fragments, fragment (g, c) at codes_offset +
  (g * K/64 + c) * 2048; byte 32*L + b holds the E4M3 code of packed row
  32g + L%32 at k = 64c + 32(b//16) + 16(L//32) + b%16 (two 16-element runs
  per lane).
* FP8 scales: float32 [Np] at scales_offset, in packed row order.
* MXFP8 codes: as FP8 codes (2048-byte fragments, one E4M3 byte per element).
* MXFP8 scales: as FP4 scales (128-byte records (s, g), byte 2*L + j = E8M0 scale
  of packed row 32g + L%32 for the K block 4s + 2j + L//32).
* NVFP4 codes: as FP4 codes.  NVFP4 scales: 256-byte records (s, g) at
  scales_offset + (s * Np/32 + g) * 256; byte 4*L + 2*j + b is the E4M3 scale of
  packed row 32g + L%32 for the 16-element K block 8s + 4j + 2(L//32) + b.  The
  fp32 tensor scale sits in the header at byte 56.
"""
from __future__ import annotations

import numpy as np

MAGIC = 0x51544944
HEADER = 256
FMT_FP4, FMT_FP8, FMT_MX8, FMT_NV4 = 1, 2, 3, 4
EPI_IDENTITY, EPI_GATED_SILU, EPI_QK_RMSNORM = 0, 1, 2


def padded_rows(N: int) -> int:
    return (N + 255) // 256 * 256


def row_perm(epi: int, N: int, Np: int) -> np.ndarray:
    """Logical weight row held by each packed row (-1 for padding)."""
    p = np.arange(Np)
    if epi == EPI_GATED_SILU:
        P, i = p // 64, p % 64
        logical = np.where(i < 32, 32 * P + i, N // 2 + 32 * P + (i - 32))
    else:
        logical = p.copy()
    return np.where(p < N, logical, -1)


def read_header(blob: np.ndarray) -> dict:
    b = np.asarray(blob, dtype=np.uint8)
    u32 = b[:32].view(np.uint32)
    u64 = b[32:56].view(np.uint64)
    return {"magic": int(u32[0]), "version": int(u32[1]), "fmt": int(u32[2]), "epi": int(u32[3]),
            "N": int(u32[4]), "K": int(u32[5]), "Np": int(u32[6]),
            "codes_offset": int(u64[0]), "scales_offset": int(u64[1]), "total": int(u64[2])}


def decode(blob: np.ndarray, fmt: int, epi: int, N: int, K: int):
    """Return (codes, scales) in logical row order.

    FP4: codes uint8 [N, K/2] (low nibble = even k), scales uint8 [N, K/32].
    FP8: codes uint8 [N, K], scales float32 [N].
    MXFP8: codes uint8 [N, K], scales uint8 [N, K/32].
    NVFP4: codes uint8 [N, K/2], scales uint8 [N, K/16] (the tensor scale is
    ``tensor_scale(blob)``).
    """
    b = np.asarray(blob, dtype=np.uint8)
    Np = padded_rows(N)
    G = Np // 32
    perm = row_perm(epi, N, Np)
    if fmt in (FMT_FP4, FMT_NV4):
        cbytes = Np * K // 2
        frag = b[HEADER:HEADER + cbytes].reshape(G, K // 64, 64, 16)        # [g][c][L][b]
        rows = np.empty((Np, K // 2), dtype=np.uint8)
        for L in range(64):
            r = np.arange(G) * 32 + L % 32
            col0 = (L // 32) * 16                                            # byte offset in the 32-byte chunk
            for c in range(K // 64):
                rows[r, c * 32 + col0:c * 32 + col0 + 16] = frag[:, c, L, :]
    elif fmt in (FMT_FP8, FMT_MX8):
        cbytes = Np * K
        frag = b[HEADER:HEADER + cbytes].reshape(G, K // 64, 64, 32)
        rows = np.empty((Np, K), dtype=np.uint8)
        for L in range(64):
            r = np.arange(G) * 32 + L % 32
            for c in range(K // 64):
                for run in range(2):                                         # bytes 16*run .. 16*run + 15
                    k0 = c * 64 + 32 * run + 16 * (L // 32)
                    rows[r, k0:k0 + 16] = frag[:, c, L, 16 * run:16 * run + 16]
    else:
        raise ValueError("unknown format")
    if fmt == FMT_FP8:
        sc = b[HEADER + cbytes:HEADER + cbytes + 4 * Np].copy().view(np.float32)
    elif fmt == FMT_NV4:
        sbytes = Np * K // 16
        sg = b[HEADER + cbytes:HEADER + cbytes + sbytes].reshape(K // 128, G, 64, 2, 2)   # [s][g][L][j][b]
        sc = np.empty((Np, K // 16), dtype=np.uint8)
        for L in range(64):
            r = np.arange(G) * 32 + L % 32
            for s in range(K // 128):
                for j in range(2):
                    for bb in range(2):
                        sc[r, 8 * s + 4 * j + 2 * (L // 32) + bb] = sg[s, :, L, j, bb]
    else:
        sbytes = Np * K // 32
        sg = b[HEADER + cbytes:HEADER + cbytes + sbytes].reshape(K // 128, G, 64, 2)   # [s][g][L][j]
        sc = np.empty((Np, K // 32), dtype=np.uint8)
        for L in range(64):
            r = np.arange(G) * 32 + L % 32
            for s in range(K // 128):
                for j in range(2):
                    sc[r, 4 * s + 2 * j + L // 32] = sg[s, :, L, j]
    codes = np.zeros((N,) + rows.shape[1:], dtype=rows.dtype)
    scales = np.zeros((N,) + sc.shape[1:], dtype=sc.dtype)
    valid = perm >= 0
    codes[perm[valid]] = rows[valid]
    scales[perm[valid]] = sc[valid]
    padding = {"codes": rows[~valid], "scales": sc[~valid]}
    return codes, scales, padding


def tensor_scale(blob: np.ndarray) -> np.float32:
    """The NVFP4 blob's fp32 tensor scale (header byte 56)."""
    return np.asarray(blob, dtype=np.uint8)[56:60].copy().view(np.float32)[0]
