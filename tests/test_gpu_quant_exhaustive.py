"""Exhaustive GPU parity of the block-scaled quantizers: every finite bf16 value
under every scale byte it can meet.

The scale byte of a 32-element block follows from the block's largest magnitude
(FP4: clamp(floor(log2 amax) - 2 + 127, 0, 254); MXFP8: the same with 8 for E4M3's
largest exponent).  For each reachable byte e the sweep builds blocks whose
maximum is the largest bf16 magnitude with that byte, and fills the other 31
elements with every finite bf16 value no larger in magnitude (both signs): every
value that can share a block with scale byte e is quantized under e once.  The
kernel quantizes these blocks and its codes and scale bytes must equal the
oracle's bit for bit.  This also covers the hardware conversion the kernels use
(v_cvt_scalef32_pk_fp4_bf16, and the exact doubling path of byte 0 whose float
scale would be subnormal) on every input it can receive.

FP4: bytes 0..252, 8.4 M swept values.  MXFP8: bytes 0..246, 8.4 M values.
"""
import numpy as np
import pytest

from oracle import formats, quant
from tests.test_gpu_quant import _run_fp4, _run_mx8

K = 3072


@pytest.fixture(scope="module")
def ditq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_dit_amd
    return bit_gemm_dit_amd


def sweep_blocks(emax_elem: int, n_bytes: int, seed: int):
    """Blocks [n, 32] of bf16 bits and the scale byte each was built for."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = allb[np.isfinite(formats.bf16_to_f64(allb))]
    mag = fin & 0x7FFF
    rng = np.random.default_rng(seed)
    blocks, want = [], []
    for e in range(n_bytes):
        # the largest magnitude whose exponent field gives byte e (byte 0: every
        # exponent field up to emax_elem)
        top = ((e + emax_elem) << 7) | 0x7F if e > 0 else (emax_elem << 7) | 0x7F
        vals = rng.permutation(fin[mag <= top])
        vals = np.concatenate([vals, np.zeros((-len(vals)) % 31, np.uint16)])
        grp = vals.reshape(-1, 31)
        head = np.full((len(grp), 1), top, np.uint16) | (rng.integers(0, 2, (len(grp), 1)) << 15).astype(np.uint16)
        b = np.concatenate([grp[:, :5], head, grp[:, 5:]], axis=1)      # the maximum sits inside the block
        blocks.append(b)
        want.append(np.full(len(b), e, np.uint8))
    blocks = np.concatenate(blocks)
    want = np.concatenate(want)
    pad = (-len(blocks)) % (K // 32)
    blocks = np.concatenate([blocks, np.zeros((pad, 32), np.uint16)])
    want = np.concatenate([want, np.zeros(pad, np.uint8)])
    return blocks.reshape(-1, K), want.reshape(-1, K // 32)


def test_sweep_construction_reaches_every_byte():
    """CPU check of the sweep itself: the oracle gives each block the byte it was
    built for, and every reachable byte occurs."""
    for emax, n, fn in ((2, 253, quant.quantize_fp4), (8, 247, quant.quantize_mx8)):
        bits, want = sweep_blocks(emax, n, 0)
        _, s = fn(bits)
        np.testing.assert_array_equal(s, want)
        assert set(np.unique(want)) == set(range(n))


@pytest.mark.gpu
def test_fp4_every_bf16_under_every_scale_byte(ditq):
    bits, want = sweep_blocks(2, 253, 11)
    print(f"FP4 sweep: {bits.size} elements, {bits.shape[0]} rows", flush=True)
    c, s = _run_fp4(ditq, bits)
    rc, rs = quant.quantize_fp4(bits)
    np.testing.assert_array_equal(rs, want)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


@pytest.mark.gpu
def test_mx8_every_bf16_under_every_scale_byte(ditq):
    bits, want = sweep_blocks(8, 247, 12)
    print(f"MXFP8 sweep: {bits.size} elements, {bits.shape[0]} rows", flush=True)
    c, s = _run_mx8(ditq, bits)
    rc, rs = quant.quantize_mx8(bits)
    np.testing.assert_array_equal(rs, want)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)
