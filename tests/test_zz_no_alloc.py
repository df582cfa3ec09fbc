"""The allocation-free quantizer entry (dit_quantize_act_noalloc) against
dit_quantize_act, through the C ABI.

dit_quantize_act_noalloc keeps NVFP4's tensor-maximum work space in a static array
of the library (one per device) instead of the caller's scale buffer.  Two calls
in a row, the second on a smaller input, must each give exactly the codes, block
scales and tensor scale of dit_quantize_act on the same input: the shared array
keeps the first call's contents, and nothing of them may leak into the second.
The scale buffer given to the allocation-free entry is only M*K/16 + 16 bytes,
followed by guard bytes that must stay untouched.
"""
import numpy as np
import pytest

from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

NV4 = 4


@pytest.fixture(scope="module")
def ditq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_dit_amd
    return bit_gemm_dit_amd


def _input(M, K, seed, amax):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20.0
    x[int(rng.integers(M)), int(rng.integers(K))] = amax        # the tensor maximum
    return f32_to_bf16_bits(x)


def _reference(ditq, x, M, K):
    """dit_quantize_act (work space in the scale buffer's tail): codes, scales[:M*K/16 + 16]."""
    import torch
    st = torch.cuda.current_stream().cuda_stream
    codes = torch.empty(ditq.dit_act_code_bytes(NV4, M, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty(ditq.dit_act_scale_bytes(NV4, M, K), dtype=torch.uint8, device="cuda")
    ditq.dit_quantize_act(NV4, x.data_ptr(), M, K, K, codes.data_ptr(), scales.data_ptr(), st)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()[:M * K // 16 + 16]


def _noalloc(ditq, x, M, K, guard=256):
    import torch
    st = torch.cuda.current_stream().cuda_stream
    codes = torch.empty(ditq.dit_act_code_bytes(NV4, M, K), dtype=torch.uint8, device="cuda")
    n = M * K // 16 + 16
    scales = torch.full((n + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    ditq.dit_quantize_act_noalloc(NV4, x.data_ptr(), M, K, K, codes.data_ptr(), scales.data_ptr(), st)
    torch.cuda.synchronize()
    s = scales.cpu().numpy()
    assert np.all(s[n:] == 0xA5), "write past M*K/16 + 16 scale bytes"
    return codes.cpu().numpy(), s[:n]


def _same(got, want, M, K, label):
    gc, gs = got
    wc, ws = want
    np.testing.assert_array_equal(gc, wc, err_msg=f"{label}: codes")
    np.testing.assert_array_equal(gs[:M * K // 16], ws[:M * K // 16], err_msg=f"{label}: block scales")
    np.testing.assert_array_equal(gs[M * K // 16 + 4:M * K // 16 + 8], ws[M * K // 16 + 4:M * K // 16 + 8],
                                  err_msg=f"{label}: tensor scale")


def test_noalloc_equals_dit_quantize_act_twice_second_smaller(ditq):
    from tests.gpu_util import to_dev_bf16
    # first call: a large tensor maximum over many workgroups; second: a smaller input
    # whose maximum is far below the first one's (a stale work space would show)
    for i, (M, K, amax) in enumerate([(4608, 3072, 3000.0), (300, 512, 7.0)]):
        print(f"case noalloc call {i}: M={M} K={K}", flush=True)
        x = to_dev_bf16(_input(M, K, 100 + i, amax))
        _same(_noalloc(ditq, x, M, K), _reference(ditq, x, M, K), M, K, f"call {i}")


def test_noalloc_other_formats_are_dit_quantize_act(ditq):
    import torch
    from tests.gpu_util import to_dev_bf16
    M, K = 129, 384
    x = to_dev_bf16(_input(M, K, 7, 50.0))
    st = torch.cuda.current_stream().cuda_stream
    for fmt in (1, 2, 3):
        outs = []
        for fn in (ditq.dit_quantize_act, ditq.dit_quantize_act_noalloc):
            c = torch.empty(ditq.dit_act_code_bytes(fmt, M, K), dtype=torch.uint8, device="cuda")
            s = torch.empty(ditq.dit_act_scale_bytes(fmt, M, K), dtype=torch.uint8, device="cuda")
            fn(fmt, x.data_ptr(), M, K, K, c.data_ptr(), s.data_ptr(), st)
            torch.cuda.synchronize()
            outs.append((c.cpu().numpy(), s.cpu().numpy()))
        np.testing.assert_array_equal(outs[0][0], outs[1][0])
        np.testing.assert_array_equal(outs[0][1], outs[1][1])
