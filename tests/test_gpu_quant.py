"""GPU parity of the activation quantizers: codes and scales bit-exact against the oracle."""
import numpy as np
import pytest

from oracle import formats, quant
from workloads import f32_to_bf16_bits, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ditq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_dit_amd
    return bit_gemm_dit_amd


def _run_fp4(ditq, bits, ldx=None):
    import torch
    from tests.gpu_util import to_dev_bf16
    M, K = bits.shape
    ldx = ldx or K
    buf = np.zeros((M, ldx), dtype=np.uint16)
    buf[:, :K] = bits
    x = to_dev_bf16(buf)
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    ditq.dit_quantize_act(ditq.FMT_FP4, x.data_ptr(), M, K, ldx, codes.data_ptr(), scales.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    from tests.gpu_util import act_codes_to_rowmajor, act_scales_to_rowmajor
    return (act_codes_to_rowmajor(codes.cpu().numpy(), M, K, 1),
            act_scales_to_rowmajor(scales.cpu().numpy(), M, K))


def _special_rows(rng, M, K):
    x = rng.standard_normal((M, K)).astype(np.float32) * (2.0 ** rng.integers(-20, 20, (M, 1))).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    blocks = bits.reshape(M, K // 32, 32)
    nb = blocks.shape[0] * blocks.shape[1]
    flat = blocks.reshape(nb, 32)
    pick = rng.choice(nb, max(1, nb // 10), replace=False)
    flat[pick[0::4]] = 0                                              # zero blocks
    flat[pick[1::4], 5] = 0x8000                                      # negative zeros
    flat[pick[2::4]] = rng.integers(0, 0x0180, (len(pick[2::4]), 32)).astype(np.uint16)   # tiny / subnormal: byte 0 path
    flat[pick[3::4], 0] = 0x7F7F                                      # largest finite
    return flat.reshape(M, K)


@pytest.mark.parametrize("M,K,ldx", [(1, 256, 256), (63, 3072, 3072), (300, 512, 520), (7, 4096, 4104)])
def test_fp4_quantizer_bitexact(ditq, M, K, ldx):
    rng = np.random.default_rng(M * 7 + K)
    bits = _special_rows(rng, M, K)
    c, s = _run_fp4(ditq, bits, ldx)
    rc, rs = quant.quantize_fp4(bits)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


def test_fp4_quantizer_every_bf16_value(ditq):
    """Every finite bf16 value, each under several block maxima (incl. byte 0 and the largest)."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = allb[np.isfinite(formats.bf16_to_f64(allb))]
    rng = np.random.default_rng(0)
    rows = []
    for top in (0x0000, 0x0100, 0x0140, 0x3F80, 0x4278, 0x7F7F):       # block maxima to pair values with
        v = rng.permutation(fin)
        v = np.concatenate([v, v[: (-len(v)) % 31]])
        blk = v.reshape(-1, 31)
        mag = blk & 0x7FFF
        keep = mag.max(axis=1) <= (top & 0x7FFF) if top else np.ones(len(blk), bool)
        b = np.concatenate([np.full((len(blk), 1), top, np.uint16), blk], axis=1)
        b = np.where(keep[:, None], b, np.concatenate([np.full((len(blk), 1), 0x7F7F, np.uint16), blk], axis=1))
        rows.append(b.reshape(-1))
    flat = np.concatenate(rows)
    flat = np.concatenate([flat, np.zeros((-len(flat)) % 3072, np.uint16)])
    bits = flat.reshape(-1, 3072)
    c, s = _run_fp4(ditq, bits)
    rc, rs = quant.quantize_fp4(bits)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


def test_fp4_quantizer_full_size_workload(ditq):
    d = make_inputs("mlp_gated_silu", seed=0)
    c, s = _run_fp4(ditq, d["x"])
    rc, rs = quant.quantize_fp4(d["x"])
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


def _run_fp8(ditq, bits, ldx=None):
    import torch
    from tests.gpu_util import to_dev_bf16
    M, K = bits.shape
    ldx = ldx or K
    buf = np.zeros((M, ldx), dtype=np.uint16)
    buf[:, :K] = bits
    x = to_dev_bf16(buf)
    codes = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty((M,), dtype=torch.float32, device="cuda")
    ditq.dit_quantize_act(ditq.FMT_FP8, x.data_ptr(), M, K, ldx, codes.data_ptr(), scales.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    from tests.gpu_util import act_codes_to_rowmajor
    return act_codes_to_rowmajor(codes.cpu().numpy(), M, K, 2), scales.cpu().numpy()


# the row cache: 16 register slots up to K = 8192 (including its edges), none beyond (rows read twice)
@pytest.mark.parametrize("M,K,ldx", [(1, 256, 256), (77, 3072, 3080), (33, 8448, 8448), (5, 768, 768),
                                     (9, 4096, 4104), (5, 4352, 4352), (3, 8192, 8192)])
def test_fp8_quantizer_bitexact(ditq, M, K, ldx):
    rng = np.random.default_rng(M + K)
    x = rng.standard_normal((M, K)).astype(np.float32) * (2.0 ** rng.integers(-30, 30, (M, 1))).astype(np.float32)
    x[:, rng.choice(K, K // 100 + 1, replace=False)] *= 20
    bits = f32_to_bf16_bits(x)
    bits[0, : K // 2] = 0
    if M > 2:
        bits[2, :] = 0
        bits[2, 3] = 0x8000
    c, s = _run_fp8(ditq, bits, ldx)
    rc, rs = quant.quantize_fp8(bits)
    np.testing.assert_array_equal(s.view(np.uint32), rs.view(np.uint32))
    np.testing.assert_array_equal(c, rc)


def test_fp8_quantizer_full_size_workload(ditq):
    d = make_inputs("fp8_cfg_pair", seed=0)
    c, s = _run_fp8(ditq, d["x"])
    rc, rs = quant.quantize_fp8(d["x"])
    np.testing.assert_array_equal(s.view(np.uint32), rs.view(np.uint32))
    np.testing.assert_array_equal(c, rc)


def _run_mx8(ditq, bits, ldx=None):
    import torch
    from tests.gpu_util import act_codes_to_rowmajor, act_scales_to_rowmajor, to_dev_bf16
    M, K = bits.shape
    ldx = ldx or K
    buf = np.zeros((M, ldx), dtype=np.uint16)
    buf[:, :K] = bits
    x = to_dev_bf16(buf)
    codes = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    ditq.dit_quantize_act(ditq.FMT_MX8, x.data_ptr(), M, K, ldx, codes.data_ptr(), scales.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return (act_codes_to_rowmajor(codes.cpu().numpy(), M, K, 2),
            act_scales_to_rowmajor(scales.cpu().numpy(), M, K))


@pytest.mark.parametrize("M,K,ldx", [(1, 256, 256), (63, 3072, 3072), (300, 512, 520), (7, 4096, 4104)])
def test_mx8_quantizer_bitexact(ditq, M, K, ldx):
    rng = np.random.default_rng(M * 11 + K)
    bits = _special_rows(rng, M, K)
    c, s = _run_mx8(ditq, bits, ldx)
    rc, rs = quant.quantize_mx8(bits)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


def test_mx8_quantizer_every_bf16_value(ditq):
    """Every finite bf16 value, each under several block maxima: byte 0 (maxima
    with exponent field <= 8, where products reach fp32's subnormal range), the
    first non-zero bytes, ordinary and the largest maxima."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = allb[np.isfinite(formats.bf16_to_f64(allb))]
    rng = np.random.default_rng(1)
    rows = []
    for top in (0x0000, 0x0400, 0x0480, 0x04FF, 0x3F80, 0x43E0, 0x4278, 0x7F7F):
        v = rng.permutation(fin)
        v = np.concatenate([v, v[: (-len(v)) % 31]])
        blk = v.reshape(-1, 31)
        mag = blk & 0x7FFF
        keep = mag.max(axis=1) <= (top & 0x7FFF) if top else np.ones(len(blk), bool)
        b = np.concatenate([np.full((len(blk), 1), top, np.uint16), blk], axis=1)
        b = np.where(keep[:, None], b, np.concatenate([np.full((len(blk), 1), 0x7F7F, np.uint16), blk], axis=1))
        rows.append(b.reshape(-1))
    flat = np.concatenate(rows)
    flat = np.concatenate([flat, np.zeros((-len(flat)) % 3072, np.uint16)])
    bits = flat.reshape(-1, 3072)
    c, s = _run_mx8(ditq, bits)
    rc, rs = quant.quantize_mx8(bits)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


def test_mx8_quantizer_full_size_workload(ditq):
    d = make_inputs("mlp_gated_silu", seed=0)
    c, s = _run_mx8(ditq, d["x"])
    rc, rs = quant.quantize_mx8(d["x"])
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


def _run_nv4(ditq, bits, ldx=None):
    import torch
    from tests.gpu_util import act_codes_to_rowmajor, nv4_act_scales, to_dev_bf16
    M, K = bits.shape
    ldx = ldx or K
    buf = np.zeros((M, ldx), dtype=np.uint16)
    buf[:, :K] = bits
    x = to_dev_bf16(buf)
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.full((ditq.dit_act_scale_bytes(ditq.FMT_NV4, M, K),), 0xAB, dtype=torch.uint8, device="cuda")
    ditq.dit_quantize_act(ditq.FMT_NV4, x.data_ptr(), M, K, ldx, codes.data_ptr(), scales.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    blocks, st = nv4_act_scales(scales.cpu().numpy(), M, K)
    return act_codes_to_rowmajor(codes.cpu().numpy(), M, K, 1), blocks, st


@pytest.mark.parametrize("M,K,ldx", [(1, 256, 256), (63, 3072, 3072), (300, 512, 520), (7, 4096, 4104)])
def test_nv4_quantizer_bitexact(ditq, M, K, ldx):
    rng = np.random.default_rng(M * 13 + K)
    bits = _special_rows(rng, M, K)
    c, s, st = _run_nv4(ditq, bits, ldx)
    rc, rs, rst = quant.quantize_nv4(bits)
    assert np.float32(st).view(np.uint32) == np.float32(rst).view(np.uint32)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


def test_nv4_quantizer_every_bf16_value(ditq):
    """Every finite bf16 value (hence every block-scale and element rounding case the
    tensor's scale allows), twice: once in a tensor whose maximum is bf16's largest
    value, once in small-magnitude blocks under a tensor maximum of 1."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = allb[np.isfinite(formats.bf16_to_f64(allb))]
    rng = np.random.default_rng(2)
    v = rng.permutation(fin)
    v = np.concatenate([v, np.zeros((-len(v)) % 3072, np.uint16)])
    for bits in (v.reshape(-1, 3072), np.where((v & 0x7FFF) <= 0x3F80, v, v & 0x803F).reshape(-1, 3072)):
        c, s, st = _run_nv4(ditq, bits)
        rc, rs, rst = quant.quantize_nv4(bits)
        assert np.float32(st).view(np.uint32) == np.float32(rst).view(np.uint32)
        np.testing.assert_array_equal(s, rs)
        np.testing.assert_array_equal(c, rc)


@pytest.mark.parametrize("where", ["first", "last", "interior"])
def test_nv4_tensor_maximum_anywhere(ditq, where):
    """The tensor maximum is found wherever the one largest magnitude sits: the first
    element, the last, or a random one inside.  The shape spans more than one
    grid-stride pass of the maximum kernel, and the row stride is padded (the
    padding holds a larger value that must be ignored)."""
    import torch
    from tests.gpu_util import to_dev_bf16
    M, K, ldx = 4608, 3072, 3080
    rng = np.random.default_rng({"first": 1, "last": 2, "interior": 3}[where])
    bits = f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    r, c = {"first": (0, 0), "last": (M - 1, K - 1)}.get(where, (int(rng.integers(M)), int(rng.integers(K))))
    bits[r, c] = f32_to_bf16_bits(np.array([-1000.0 if where == "interior" else 1000.0], np.float32))[0]
    buf = np.full((M, ldx), f32_to_bf16_bits(np.array([30000.0], np.float32))[0], dtype=np.uint16)
    buf[:, :K] = bits
    x = to_dev_bf16(buf)
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((ditq.dit_act_scale_bytes(ditq.FMT_NV4, M, K),), dtype=torch.uint8, device="cuda")
    print(f"nv4 tensor maximum at {where} ({r}, {c})", flush=True)
    ditq.dit_quantize_act(ditq.FMT_NV4, x.data_ptr(), M, K, ldx, codes.data_ptr(), scales.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    from tests.gpu_util import nv4_act_scales
    _, st = nv4_act_scales(scales.cpu().numpy(), M, K)
    want = quant.nv4_tensor_scale(np.float32(1000.0))
    assert np.float32(st).view(np.uint32) == np.float32(want).view(np.uint32)


def test_nv4_quantizer_full_size_workload(ditq):
    d = make_inputs("mlp_gated_silu", seed=0)
    c, s, st = _run_nv4(ditq, d["x"])
    rc, rs, rst = quant.quantize_nv4(d["x"])
    assert np.float32(st) == rst
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)
