"""Quantizers of the low-bit DiT linear layer (CPU oracle, float64 / exact).

Test infrastructure (see the package docstring).

FP4 path (page "How fal made Ideogram V4 6x faster", paragraph 2: the DiT runs
in a 4-bit float format; page "Versnellende diffusiemodellen met TheStage AI",
section on acceleration and compression: activation statistics change from one
diffusion iteration to the next, so activation scales are computed on the fly
rather than calibrated once):

  per row r and per block b of 32 consecutive K elements
    amax  = max |x| over the block (exact)
    byte  = clamp(floor(log2 amax) - 2 + 127, 0, 254)      (E8M0 scale, 2**(byte-127));
            byte = 0 when amax == 0.  The "-2" is the exponent of E2M1's
            largest magnitude (6 = 1.5 * 2**2), so the block maximum lands in [4, 8).
    v     = x * 2**-(byte - 127)                             (exact)
    code  = sign(x) | RNE_E2M1(min(|v|, 6))                  ties to the even mantissa bit;
            the sign bit is copied from x even when the magnitude rounds to 0.
    codes are packed two per byte, the even k in the low nibble.

FP8 path (page "WaveSpeedAI X DataCrunch: FLUX real-time image inference on
B200", engine list: BF16/FP8 mixed precision; page on FLUX.1-dev LoRA inference
(aitime.ge): FP8 is lossy but the best speed/memory trade-off):

  per activation row (per weight row n = output column n), in IEEE fp32:
    amax = max |x|,  s = fl32(amax / 448)  (s = 1 when amax == 0)
    q    = RNE_E4M3(fl32(x / s))           OCP E4M3, saturating at 448, sign kept.

MXFP8 path (FP8 as the safer precision, pages above; the block structure of the
4-bit path, so both formats run through the same block-scaled matrix units):

  per row r and per block b of 32 consecutive K elements
    amax  = max |x| over the block (exact)
    byte  = clamp(floor(log2 amax) - 8 + 127, 0, 254)      (E8M0 scale); 0 when amax == 0.
            The "-8" is the exponent of E4M3's largest magnitude (448 = 1.75 * 2**8),
            so the block maximum lands in [256, 512) and (448, 512) clips to 448.
    v     = x * 2**-(byte - 127)                             (exact)
    code  = RNE_E4M3(v), saturating at 448, sign kept.

NVFP4 path (the format page "How fal made Ideogram V4 6x faster" names in
paragraph 2: a 4-bit float with two levels of scaling, E4M3 scales per 16
elements and one fp32 scale per tensor), every step an IEEE fp32 operation:

  s_t   = fl32(amax_tensor / 2688)  (2688 = 6 * 448; s_t = 1 when the tensor is zero)
  per row and per block of 16 consecutive K elements:
    d   = fl32(amax_block / fl32(6 * s_t))
    s_b = RNE_E4M3(min(d, 448))                                 (the stored scale code)
    q   = sign(x) | RNE_E2M1(min(|fl32(x / fl32(dec(s_b) * s_t))|, 6)),  magnitude 0 when s_b = 0
  value = E2M1(q) * dec(s_b) * s_t.

Every rounding function below exists twice (a closed-form threshold rule and a
brute-force nearest-point search); the tests require them to agree on every
input class.
"""
from __future__ import annotations

import numpy as np

from . import formats

FP4_BLOCK = 32
MX_BLOCK = 32
E2M1_EMAX = 2            # largest E2M1 magnitude is 6 = 1.5 * 2**2
E4M3_EMAX = 8            # largest E4M3 magnitude is 448 = 1.75 * 2**8
E4M3_MAX = 448.0


def _check_finite(v: np.ndarray) -> None:
    if not np.all(np.isfinite(v)):
        raise ValueError("the quantizers are defined for finite inputs only")


# ---------------------------------------------------------------- FP4 scale rule
def fp4_scale_byte(amax: np.ndarray) -> np.ndarray:
    """E8M0 scale byte of a block whose exact maximum magnitude is ``amax`` (float64).

    floor(log2 amax) is read off frexp (amax = f * 2**ex, f in [0.5, 1)), which is
    exact for every float64, so the rule is integer-exact.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    e = ex.astype(np.int64) - 1 - E2M1_EMAX
    byte = np.clip(e + 127, 0, 254)
    return np.where(amax == 0, 0, byte).astype(np.uint8)


# ---------------------------------------------------------------- E2M1 rounding
def e2m1_rne_threshold(a: np.ndarray) -> np.ndarray:
    """Magnitude code (0..7) of |v| = a >= 0, rounded to nearest, ties to even.

    Grid: 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7).  The midpoints between
    neighbours are .25, .75, 1.25, 1.75, 2.5, 3.5, 5.  At a midpoint the code with
    mantissa bit 0 wins: .25 -> 0, .75 -> 2, 1.25 -> 2, 1.75 -> 4, 2.5 -> 4,
    3.5 -> 6, 5 -> 6.  So the count of midpoints passed uses ">" where the lower
    neighbour is even and ">=" where the upper one is.  Above 6 everything maps to
    6 (saturation: E2M1 has no infinity).
    """
    a = np.asarray(a, dtype=np.float64)
    c = ((a > 0.25).astype(np.int64) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
         + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    return c.astype(np.uint8)


def e2m1_rne_bruteforce(a: np.ndarray) -> np.ndarray:
    """Same rounding by search: the grid point at the least distance; on a tie the
    candidate whose code has mantissa bit (code & 1) equal to 0.  Magnitudes above
    6 are nearest to 6, which is the saturation rule."""
    # Clamping at 8 changes nothing mathematically (everything above 6 is nearest to
    # 6) but keeps float64 from absorbing the grid offsets for huge magnitudes, where
    # all eight distances would compare equal.
    a = np.minimum(np.asarray(a, dtype=np.float64), 8.0)
    grid = formats.E2M1_GRID
    d = np.abs(a[..., None] - grid)                       # [..., 8]
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among the tied candidates prefer an even code; there are at most two ties
    even = cand & ((np.arange(8) & 1) == 0)
    pick = np.where(even.any(axis=-1, keepdims=True), even, cand)
    return np.argmax(pick, axis=-1).astype(np.uint8)


# ---------------------------------------------------------------- FP4 quantizer
def quantize_fp4(x_bits: np.ndarray, rounding=e2m1_rne_threshold):
    """Quantize bf16 rows [R, K] (uint16 bits) to FP4 E2M1 with E8M0 block-32 scales.

    Returns ``codes`` uint8 [R, K/2] (low nibble = even k) and ``scales`` uint8
    [R, K/32].  K must be a multiple of 32.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, K = x_bits.shape
    if K % FP4_BLOCK:
        raise ValueError("K must be a multiple of 32")
    x = formats.bf16_to_f64(x_bits)
    _check_finite(x)
    xb = x.reshape(R, K // FP4_BLOCK, FP4_BLOCK)
    amax = np.abs(xb).max(axis=-1)
    scales = fp4_scale_byte(amax)
    v = xb * np.ldexp(1.0, 127 - scales.astype(np.int64))[..., None]     # exact power-of-two scaling
    mag = rounding(np.abs(v)).reshape(R, K)
    sign = ((x_bits >> 15) & 1).astype(np.uint8)
    code = mag | (sign << 3)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales


def unpack_fp4_codes(packed: np.ndarray) -> np.ndarray:
    """[R, K/2] bytes -> [R, K] 4-bit codes (even k from the low nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def dequantize_fp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = unpack_fp4_codes(packed)
    R, K = codes.shape
    vals = formats.e2m1_decode(codes).reshape(R, K // FP4_BLOCK, FP4_BLOCK)
    return (vals * formats.e8m0_decode(scales)[..., None]).reshape(R, K)


# ---------------------------------------------------------------- E4M3 rounding
def e4m3_rne_fields(y: np.ndarray) -> np.ndarray:
    """fp32 values -> OCP E4M3 codes, rounding to nearest even, from the fields.

    For |y| >= 2**-6 (normal E4M3) the exponent E = floor(log2|y|) keeps 3 mantissa
    bits: q = RNE(|y| / 2**(E-3)) in [8, 16]; q == 16 carries into the exponent.
    Below 2**-6 the spacing is the subnormal step 2**-9: q = RNE(|y| / 2**-9),
    and q == 8 is exactly the smallest normal (code 0x08), so code == q there.
    Magnitudes above 448 saturate to 448 (0x7E); the sign bit is copied from y.
    """
    y = np.asarray(y, dtype=np.float32)
    _check_finite(y)
    a = np.abs(y.astype(np.float64))
    sign = ((y.view(np.uint32) >> 31) & 1).astype(np.int64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    E = ex.astype(np.int64) - 1
    normal = a >= 2.0 ** -6
    qn = np.rint(a / np.ldexp(1.0, E - 3)).astype(np.int64)          # np.rint: half to even
    carry = qn == 16
    En = np.where(carry, E + 1, E)
    qn = np.where(carry, 8, qn)
    code_n = ((En + 7) << 3) | (qn - 8)
    code_s = np.rint(np.minimum(a, 1.0) / 2.0 ** -9).astype(np.int64)   # used only below 2**-6
    code = np.where(normal, code_n, code_s)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.minimum(code, 0x7E)
    return (code | (sign << 7)).astype(np.uint8)


def e4m3_rne_bruteforce(y: np.ndarray) -> np.ndarray:
    """Same rounding by search over the 127 non-negative E4M3 values (index = code):
    nearest value, ties to the even code (mantissa bit 0); above 448 the nearest
    finite value is 448."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    table = formats.E4M3_POS
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    dlo = np.abs(a - table[lo])
    dhi = np.abs(table[hi] - a)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    sign = ((y.view(np.uint32) >> 31) & 1).astype(np.int64)
    return (pick.astype(np.int64) | (sign << 7)).astype(np.uint8)


# ---------------------------------------------------------------- FP8 quantizer
def fp8_row_scale(amax_f32: np.ndarray) -> np.ndarray:
    """s = fl32(amax / 448), an IEEE fp32 division; 1.0 for an all-zero row."""
    amax_f32 = np.asarray(amax_f32, dtype=np.float32)
    s = (amax_f32 / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(amax_f32 == 0, np.float32(1.0), s).astype(np.float32)


def quantize_fp8(x_bits: np.ndarray, rounding=e4m3_rne_fields):
    """Quantize bf16 rows [R, K] to E4M3 codes [R, K] with one fp32 scale per row [R]."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    x = (x_bits.astype(np.uint32) << 16).view(np.float32)
    _check_finite(x)
    amax = np.abs(x).max(axis=1)
    s = fp8_row_scale(amax)
    y = (x / s[:, None]).astype(np.float32)               # IEEE fp32 division, correctly rounded
    return rounding(y), s


def dequantize_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return formats.e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]


# ---------------------------------------------------------------- MXFP8 quantizer
def mx8_scale_byte(amax: np.ndarray) -> np.ndarray:
    """E8M0 scale byte of an MXFP8 block with exact maximum magnitude ``amax``:
    clamp(floor(log2 amax) - 8 + 127, 0, 254), 0 for an all-zero block.  floor(log2)
    is read off frexp, exact for every float64."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    e = ex.astype(np.int64) - 1 - E4M3_EMAX
    byte = np.clip(e + 127, 0, 254)
    return np.where(amax == 0, 0, byte).astype(np.uint8)


def quantize_mx8(x_bits: np.ndarray, rounding=e4m3_rne_fields):
    """Quantize bf16 rows [R, K] (uint16 bits) to E4M3 codes [R, K] with one E8M0
    scale per 32-element K block, [R, K/32].

    v = x * 2**(127 - byte) is exact in float64.  The rounding functions take fp32;
    the conversion is exact for every |v| >= 2**-126 (a bf16 significand times a
    power of two) and below that only moves values that lie far under E4M3's
    smallest rounding threshold 2**-10, whose code is a signed zero either way.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, K = x_bits.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    x = formats.bf16_to_f64(x_bits)
    _check_finite(x)
    xb = x.reshape(R, K // MX_BLOCK, MX_BLOCK)
    scales = mx8_scale_byte(np.abs(xb).max(axis=-1))
    v = xb * np.ldexp(1.0, 127 - scales.astype(np.int64))[..., None]
    codes = rounding(v.reshape(R, K).astype(np.float32))
    return codes, scales


def dequantize_mx8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    R, K = c.shape
    vals = formats.e4m3_decode(c).reshape(R, K // MX_BLOCK, MX_BLOCK)
    return (vals * formats.e8m0_decode(scales)[..., None]).reshape(R, K)


# ---------------------------------------------------------------- NVFP4 quantizer
NV_BLOCK = 16
NV_TENSOR_DIV = 2688.0        # 6 * 448: the tensor maximum maps to the largest code times the largest scale


def nv4_tensor_scale(amax_f32) -> np.float32:
    """s_t = fl32(amax / 2688), 1 for an all-zero tensor."""
    a = np.float32(amax_f32)
    return np.float32(1.0) if a == 0 else np.float32(a / np.float32(NV_TENSOR_DIV))


def quantize_nv4(x_bits: np.ndarray, rounding=e2m1_rne_threshold, scale_rounding=e4m3_rne_fields):
    """Quantize a bf16 tensor [R, K] to NVFP4.

    Returns ``codes`` uint8 [R, K/2] (two E2M1 codes per byte, even k in the low
    nibble), ``scales`` uint8 [R, K/16] (E4M3 block scale codes) and ``s_t``
    (float32 tensor scale).  K must be a multiple of 16.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, K = x_bits.shape
    if K % NV_BLOCK:
        raise ValueError("K must be a multiple of 16")
    x = (x_bits.astype(np.uint32) << 16).view(np.float32)
    _check_finite(x)
    s_t = nv4_tensor_scale(np.abs(x).max() if x.size else 0.0)
    six_st = np.float32(np.float32(6.0) * s_t)
    xb = x.reshape(R, K // NV_BLOCK, NV_BLOCK)
    d = (np.abs(xb).max(axis=-1) / six_st).astype(np.float32)
    scales = scale_rounding(np.minimum(d, np.float32(E4M3_MAX)))
    denom = (formats.e4m3_decode(scales).astype(np.float32) * s_t).astype(np.float32)      # fl32(dec(s_b) * s_t)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (xb / denom[..., None]).astype(np.float32)
    y = np.where(denom[..., None] == 0, np.float32(0.0), y)
    mag = rounding(np.minimum(np.abs(y.astype(np.float64)), 6.0)).reshape(R, K)
    sign = ((x_bits >> 15) & 1).astype(np.uint8)
    code = mag | (sign << 3)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales, s_t


def dequantize_nv4(packed: np.ndarray, scales: np.ndarray, s_t) -> np.ndarray:
    codes = unpack_fp4_codes(packed)
    R, K = codes.shape
    vals = formats.e2m1_decode(codes).reshape(R, K // NV_BLOCK, NV_BLOCK)
    return (vals * formats.e4m3_decode(scales)[..., None]).reshape(R, K) * float(np.float32(s_t))
