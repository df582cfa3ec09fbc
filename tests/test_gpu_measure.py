"""GPU tests of the measurement kernels, through the C ABI.

The separate gated-SiLU pass (the unfused form of the gated-SiLU epilogue) is
compared element by element with the oracle's gated-SiLU of the same bf16 input:
fp32 with the hardware exp2 and reciprocal, rounded to bf16, must lie within one
bf16 ulp of the float64 value (or 1e-30 where the true value underflows).  The
MFMA probe is checked for its bookkeeping (cycles recorded, a clock in a
plausible range, work proportional to iters).
"""
import numpy as np
import pytest

from oracle import epilogue, formats
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ditq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_dit_amd
    return bit_gemm_dit_amd


def _ulp_bf16(y):
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


@pytest.mark.parametrize("M,N,ldc,ldo,rows", [(1, 16, 16, 8, None), (300, 1024, 1032, 520, None),
                                              (37, 4096, 4096, 2048, None), (4608, 16384, 16384, 8192, 64)])
def test_gated_silu_pass_matches_oracle(ditq, M, N, ldc, ldo, rows):
    import torch
    from tests.gpu_util import to_dev_bf16, to_host_bits
    rng = np.random.default_rng(M * 7 + N)
    c_bits = f32_to_bf16_bits((rng.standard_normal((M, ldc)) * 4.0).astype(np.float32))
    # a few exact special values in the gate half: zeros, large magnitudes of both signs
    c_bits[0, :4] = f32_to_bf16_bits(np.array([0.0, -0.0, 90.0, -90.0], dtype=np.float32))
    c = to_dev_bf16(c_bits)
    out = torch.full((M, ldo), float("nan"), dtype=torch.bfloat16, device="cuda")
    print(f"gated_silu M={M} N={N} ldc={ldc} ldo={ldo}", flush=True)
    ditq.dit_gated_silu_bf16(c.data_ptr(), M, N, ldc, out.data_ptr(), ldo, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got_bits = to_host_bits(out)
    sel = np.arange(M) if rows is None else np.unique(np.concatenate([[0, M - 1], rng.choice(M, rows)]))
    y = epilogue.gated_silu(formats.bf16_to_f64(c_bits[sel, :N]))
    g = formats.bf16_to_f64(got_bits[sel, : N // 2])
    assert np.all(np.isfinite(g))
    err = np.abs(g - y)
    # one bf16 ulp; below 1e-30 the hardware's overflowing exponential gives an exact
    # zero where the float64 value is a tiny number (SiLU(-90) = -7e-38)
    bad = err > np.maximum(_ulp_bf16(y), 1e-30)
    assert not bad.any(), f"{bad.sum()} elements beyond one bf16 ulp; first {np.argwhere(bad)[0]}"
    # the padding columns of out stay untouched
    if ldo > N // 2:
        assert np.all(np.isnan(formats.bf16_to_f64(got_bits[:, N // 2:])))


def test_mfma_probe_bookkeeping(ditq):
    import torch
    wg = torch.cuda.get_device_properties(0).multi_processor_count
    times, cycles = {}, {}
    for iters in (2000, 8000):
        print(f"mfma probe workgroups={wg} iters={iters}", flush=True)
        ditq.mfma_fp4_probe(wg, 100)                       # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        out = ditq.mfma_fp4_probe(wg, iters)
        e1.record()
        torch.cuda.synchronize()
        times[iters] = e0.elapsed_time(e1) * 1e-3
        cycles[iters] = out[:, 0].cpu().numpy()
        assert np.all(cycles[iters] > 0)
    # four times the work takes about four times the cycles, and the clock is plausible
    ratio = np.median(cycles[8000]) / np.median(cycles[2000])
    assert 3.0 < ratio < 5.0, ratio
    ghz = np.median(cycles[8000]) / times[8000] / 1e9
    assert 0.5 < ghz < 3.0, ghz
