"""Number formats used by the layer, decoded exactly to float64.

Test infrastructure (see the package docstring).

The pages name the formats only ("NVFP4, a 4-bit floating-point format",
page "How fal made Ideogram V4 6x faster", paragraph 2; "FP8", page "WaveSpeedAI
X DataCrunch", engine list and spec table).  The bit layouts below are the OCP
Microscaling / OCP FP8 definitions that MI355X's scaled MFMA consumes:

* FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no inf/NaN.
  Magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* E8M0: an 8-bit exponent, value 2**(b - 127); b = 255 is NaN.
* FP8 E4M3 (OCP): 1 sign, 4 exponent (bias 7), 3 mantissa bits; subnormal
  step 2**-9; max 448; 0x7F / 0xFF are NaN; no inf.

Each format has two independent decoders (bit-field formula and enumerated
table) so that a slip in one is caught by the other.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- bf16
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values (bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):            # NaN patterns stay NaN
        return u.view(np.float32).astype(np.float64)


def bf16_to_f64_bitfield(bits: np.ndarray) -> np.ndarray:
    """Second decoder: sign/exponent/mantissa fields of bf16 (8-bit exponent, bias 127, 7 mantissa bits)."""
    b = np.asarray(bits, dtype=np.int64)
    s = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    m = (b & 0x7F).astype(np.float64)
    sub = np.ldexp(m, -133)                       # m * 2**-7 * 2**-126
    nrm = np.ldexp(128.0 + m, (e - 134).astype(np.int64))
    out = np.where(e == 0, sub, nrm)
    out = np.where(e == 0xFF, np.where(m == 0, np.inf, np.nan), out)
    return s * out


# ---------------------------------------------------------------- FP4 E2M1
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit code -> value, by table lookup on the magnitude grid; bit 3 is the sign."""
    c = np.asarray(codes, dtype=np.int64)
    mag = E2M1_GRID[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_decode_bitfield(codes: np.ndarray) -> np.ndarray:
    """Second decoder from the fields: exponent (bits 2:1, bias 1), mantissa (bit 0)."""
    c = np.asarray(codes, dtype=np.int64)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, e - 1))
    return np.where((c >> 3) & 1, -mag, mag)


# ---------------------------------------------------------------- E8M0
def e8m0_decode(b: np.ndarray) -> np.ndarray:
    bb = np.asarray(b, dtype=np.int64)
    v = np.ldexp(1.0, bb - 127)
    return np.where(bb == 255, np.nan, v)


# ---------------------------------------------------------------- FP8 E4M3 (OCP)
def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Bit-field decoder: bias 7, exponent 0 is subnormal (m/8 * 2**-6), S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(8.0 + m, e - 10))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return np.where((c >> 7) & 1, -mag, mag)


def _e4m3_positive_table() -> np.ndarray:
    """Enumerate the non-negative E4M3 values in code order 0x00..0x7E.

    Built by walking the binades: 8 subnormals spaced 2**-9, then each binade
    2**(E-7) .. 2**(E-6) holds 8 values spaced 2**(E-10).
    """
    vals = [k * 2.0 ** -9 for k in range(8)]
    for E in range(1, 16):
        step = 2.0 ** (E - 10)
        base = 2.0 ** (E - 7)
        for k in range(8):
            if E == 15 and k == 7:
                break                  # NaN slot
            vals.append(base + k * step)
    return np.array(vals)


E4M3_POS = _e4m3_positive_table()          # 127 entries, index == code
E4M3_MAX = 448.0


def e4m3_decode_table(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    idx = c & 0x7F
    mag = np.where(idx == 0x7F, np.nan, E4M3_POS[np.minimum(idx, 126)])
    return np.where(c & 0x80, -mag, mag)
