"""The hot path at the largest activation the ABI accepts.

The activation code buffer must stay below 2^31 bytes: (M + 256) * (K/2 for FP4,
K for FP8) < 2^31.  At K = 256 that is M = 16,776,959 token rows for FP4 (an
8.6 GB bf16 input, a 4.3 GB gated output) and 8,388,351 for FP8.  Every byte
offset of the code and scale buffers, and the output's row offsets beyond 4 GB,
are then at the edge of their range.  The input is drawn on the GPU from a seeded
generator; sampled rows (the first and last, whose codes open and close every K
panel, and random ones) are copied back and checked against the oracle: the quantized
codes and scales bit for bit, the GEMM output within the bf16 tolerance.  One row
more is refused (DIT_EUNSUPPORTED).
"""
import numpy as np
import pytest

from oracle import layer, quant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ditq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_dit_amd
    return bit_gemm_dit_amd


@pytest.mark.parametrize("fmt_name,epi_name,N", [("fp4", "gated_silu", 256), ("fp8", "identity", 256)])
def test_largest_accepted_activation(ditq, fmt_name, epi_name, N):
    import torch
    from tests.gpu_util import compare_bf16, to_dev_bf16, to_host_bits
    from workloads import make_inputs
    fmt = {"fp4": ditq.FMT_FP4, "fp8": ditq.FMT_FP8}[fmt_name]
    epi = {"gated_silu": ditq.EPI_GATED_SILU, "identity": ditq.EPI_IDENTITY}[epi_name]
    K = 256
    row_bytes = K // 2 if fmt_name == "fp4" else K
    M = (1 << 31) // row_bytes - 256 - 1
    assert (M + 256) * row_bytes < (1 << 31) <= (M + 257) * row_bytes
    assert ditq.dit_act_code_bytes(fmt, M, K) == M * row_bytes
    width = N // 2 if epi_name == "gated_silu" else N

    d = make_inputs("tiny_gated_silu", seed=3, M=64, N=N, K=K)      # the weights (and their recipe)
    w = to_dev_bf16(d["w"])
    blob = ditq.pack_weights(w, fmt, epi)
    print(f"max-size {fmt_name} {epi_name}: M={M} N={N} K={K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    codes, scales = ditq.quantize_act(x, fmt)
    out = ditq.gemm(codes, scales, blob, N, K, fmt, epi)
    torch.cuda.synchronize()
    assert out.shape == (M, width)

    rng = np.random.default_rng(5)
    # row m's codes sit at byte (p*M + m)*64 of K panel p: the first and last rows
    # hold the first and last bytes of every panel, up to the 2^31 limit
    rows = np.unique(np.concatenate([[0, 1, M // 2, M - 257, M - 2, M - 1], rng.integers(0, M, 24)]))
    idx = torch.from_numpy(rows).cuda()
    x_rows = to_host_bits(x.index_select(0, idx))
    got = to_host_bits(out.index_select(0, idx))
    if fmt_name == "fp4":
        # panel-major codes [K/128][M][64] and scales [K/128][M][4] -> the sampled rows, row-major
        c = codes.index_select(1, idx).permute(1, 0, 2).reshape(len(rows), K // 2).cpu().numpy()
        s = scales.index_select(1, idx).permute(1, 0, 2).reshape(len(rows), K // 32).cpu().numpy()
        rc, rs = quant.quantize_fp4(x_rows)
        assert np.array_equal(c, rc) and np.array_equal(s, rs), "FP4 codes or scales differ from the oracle"
    else:
        c = codes.index_select(1, idx).permute(1, 0, 2).reshape(len(rows), K).cpu().numpy()
        s = scales.index_select(0, idx).cpu().numpy()
        rc, rs = quant.quantize_fp8(x_rows)
        assert np.array_equal(c, rc) and np.array_equal(s.view(np.uint32), np.asarray(rs, np.float32).view(np.uint32)), \
            "FP8 codes or scales differ from the oracle"
    y = layer.forward(x_rows, d["w"], fmt_name, epi_name)
    compare_bf16(got, y, f"max-size {fmt_name} rows {rows[:4]}...")
    del x, codes, scales, out
    torch.cuda.empty_cache()
    # one row more is refused before any HIP call
    assert ditq._lib.dit_quantize_act(fmt, 0x10000, M + 1, K, K, 0x20000, 0x30000, None) == 2
