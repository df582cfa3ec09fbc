"""GPU parity of the weight packer: the blob, decoded from its documented layout
by the oracle's reader, holds exactly the oracle's codes and scales."""
import numpy as np
import pytest

from oracle import packed, quant
from workloads import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ditq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_dit_amd
    return bit_gemm_dit_amd


def _pack(ditq, bits, fmt, epi, ldw=None):
    import torch
    from tests.gpu_util import to_dev_bf16
    N, K = bits.shape
    ldw = ldw or K
    buf = np.zeros((N, ldw), dtype=np.uint16)
    buf[:, :K] = bits
    w = to_dev_bf16(buf)
    nbytes = ditq.dit_packed_weight_bytes(fmt, epi, N, K)
    blob = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")      # poison: padding must be written
    ditq.dit_pack_weights(fmt, epi, w.data_ptr(), N, K, ldw, blob.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return blob.cpu().numpy()


@pytest.mark.parametrize("N,K,epi,ldw", [(512, 256, 1, 256), (320, 256, 0, 264), (128, 768, 2, 768),
                                         (1024, 512, 1, 512)])
def test_fp4_pack_bitexact(ditq, N, K, epi, ldw):
    d = make_inputs("qkv_rmsnorm_hd128", seed=N, M=1, N=N, K=K)
    blob = _pack(ditq, d["w"], 1, epi, ldw)
    hdr = packed.read_header(blob)
    assert (hdr["magic"], hdr["version"], hdr["fmt"], hdr["epi"], hdr["N"], hdr["K"]) == (packed.MAGIC, 2, 1, epi, N, K)
    assert hdr["total"] == blob.size
    c, s, pad = packed.decode(blob, 1, epi, N, K)
    rc, rs = quant.quantize_fp4(d["w"])
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)
    assert not pad["codes"].any() and not pad["scales"].any()


@pytest.mark.parametrize("name,epi", [("mlp_gated_silu", 1), ("qkv_rmsnorm_hd256", 2)])
def test_fp4_pack_full_size(ditq, name, epi):
    d = make_inputs(name, seed=0, M=1)
    N, K = d["w"].shape
    blob = _pack(ditq, d["w"], 1, epi)
    c, s, _ = packed.decode(blob, 1, epi, N, K)
    rc, rs = quant.quantize_fp4(d["w"])
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


@pytest.mark.parametrize("N,K,epi", [(320, 256, 0), (256, 512, 1), (12288, 3072, 1)])
def test_fp8_pack_bitexact(ditq, N, K, epi):
    d = make_inputs("fp8_cfg_pair", seed=N, M=1, N=N, K=K)
    d["w"][3, :] = 0                                                   # an all-zero row
    blob = _pack(ditq, d["w"], 2, epi)
    hdr = packed.read_header(blob)
    assert (hdr["magic"], hdr["fmt"], hdr["epi"], hdr["N"], hdr["K"]) == (packed.MAGIC, 2, epi, N, K)
    c, s, pad = packed.decode(blob, 2, epi, N, K)
    rc, rs = quant.quantize_fp8(d["w"])
    np.testing.assert_array_equal(s.view(np.uint32), rs.view(np.uint32))
    np.testing.assert_array_equal(c, rc)
    assert not pad["codes"].any()


@pytest.mark.parametrize("N,K,epi", [(320, 256, 0), (256, 512, 1), (384, 768, 2), (16384, 3072, 1)])
def test_mx8_pack_bitexact(ditq, N, K, epi):
    d = make_inputs("mlp_gated_silu", seed=N + 1, M=1, N=N, K=K)
    d["w"][3, :] = 0                                                   # an all-zero row
    d["w"][5, 64:96] = 0x0001                                          # a block of subnormals: byte 0
    blob = _pack(ditq, d["w"], 3, epi)
    hdr = packed.read_header(blob)
    assert (hdr["magic"], hdr["fmt"], hdr["epi"], hdr["N"], hdr["K"]) == (packed.MAGIC, 3, epi, N, K)
    assert hdr["total"] == blob.size
    c, s, pad = packed.decode(blob, 3, epi, N, K)
    rc, rs = quant.quantize_mx8(d["w"])
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)
    assert not pad["codes"].any() and not pad["scales"].any()


def test_fp8_pack_for_rmsnorm_is_the_identity_blob(ditq):
    d = make_inputs("fp8_cfg_pair", seed=9, M=1, N=384, K=256)
    a = _pack(ditq, d["w"], 2, 0)
    b = _pack(ditq, d["w"], 2, 2)
    assert packed.read_header(b)["epi"] == 2
    np.testing.assert_array_equal(a[256:], b[256:])


@pytest.mark.parametrize("N,K,epi", [(320, 256, 0), (256, 512, 1), (384, 768, 2), (16384, 3072, 1)])
def test_nv4_pack_bitexact(ditq, N, K, epi):
    d = make_inputs("mlp_gated_silu", seed=N + 2, M=1, N=N, K=K)
    d["w"][3, :] = 0                                                   # an all-zero row
    d["w"][5, 16:32] = 0x0001                                          # a block far below the tensor maximum
    blob = _pack(ditq, d["w"], 4, epi)
    hdr = packed.read_header(blob)
    assert (hdr["magic"], hdr["fmt"], hdr["epi"], hdr["N"], hdr["K"]) == (packed.MAGIC, 4, epi, N, K)
    assert hdr["total"] == blob.size
    c, s, pad = packed.decode(blob, 4, epi, N, K)
    rc, rs, rst = quant.quantize_nv4(d["w"])
    assert packed.tensor_scale(blob).view(np.uint32) == np.float32(rst).view(np.uint32)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)
    assert not pad["codes"].any() and not pad["scales"].any()


@pytest.mark.parametrize("fmt_name,epi_name", [("fp4", "gated_silu"), ("nv4", "identity")])
def test_saved_blob_reloads_to_the_same_layer(ditq, tmp_path, fmt_name, epi_name):
    """pack -> save_packed -> load_packed (header checked) gives a blob that yields the
    same GEMM output, bit for bit, as the blob it was saved from."""
    import torch
    from tests.gpu_util import to_dev_bf16
    fmt = {"fp4": ditq.FMT_FP4, "nv4": ditq.FMT_NV4}[fmt_name]
    epi = {"gated_silu": ditq.EPI_GATED_SILU, "identity": ditq.EPI_IDENTITY}[epi_name]
    d = make_inputs("tiny_gated_silu", seed=9, M=200, N=512, K=512)
    x, w = to_dev_bf16(d["x"]), to_dev_bf16(d["w"])
    blob = ditq.pack_weights(w, fmt, epi)
    path = tmp_path / "w.ditq"
    hdr = ditq.save_packed(blob, path)
    assert (hdr["fmt"], hdr["epi"], hdr["N"], hdr["K"]) == (fmt, epi, 512, 512)
    blob2 = ditq.load_packed(path, fmt=fmt, epi=epi, N=512, K=512)
    assert torch.equal(blob.cpu(), blob2.cpu())
    y1 = ditq.linear(x, blob, 512, fmt, epi)
    y2 = ditq.linear(x, blob2, 512, fmt, epi)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    with pytest.raises(ValueError):
        ditq.load_packed(path, fmt=fmt, epi=ditq.EPI_GATED_SILU if epi != ditq.EPI_GATED_SILU else ditq.EPI_IDENTITY)
