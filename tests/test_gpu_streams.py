"""Concurrent calls on different streams (the ABI allows them).

Two independent layers (different inputs, weights and buffers) are enqueued on two
streams so that their quantizers and GEMMs can overlap, several times over; each
result must equal the same layer run alone, bit for bit.  NVFP4 is included: its
quantizer keeps its tensor maximum in the caller's scale buffer, so concurrent
calls with different buffers must not see each other.
"""
import numpy as np
import pytest

from workloads import make_inputs

pytestmark = pytest.mark.gpu

FMT = {"fp4": 1, "fp8": 2, "mx8": 3, "nv4": 4}


@pytest.fixture(scope="module")
def ditq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_dit_amd
    return bit_gemm_dit_amd


@pytest.mark.parametrize("fmt_a,fmt_b", [("fp4", "fp4"), ("nv4", "nv4"), ("fp4", "mx8"), ("nv4", "fp8")])
def test_two_streams_match_sequential(ditq, fmt_a, fmt_b):
    import torch
    from tests.gpu_util import to_dev_bf16
    layers = []
    for j, fmt in enumerate((fmt_a, fmt_b)):
        d = make_inputs("mlp_gated_silu", seed=40 + j, M=1000 + 137 * j, N=2048, K=1024)
        f = FMT[fmt]
        blob = ditq.pack_weights(to_dev_bf16(d["w"]), f, ditq.EPI_GATED_SILU)
        layers.append((f, to_dev_bf16(d["x"]), blob))
    torch.cuda.synchronize()
    alone = [ditq.linear(x, blob, 2048, f, ditq.EPI_GATED_SILU).clone() for f, x, blob in layers]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    print(f"two streams: {fmt_a} + {fmt_b}", flush=True)
    for rep in range(4):
        outs = [None, None]
        torch.cuda.synchronize()
        for j in (0, 1):
            with torch.cuda.stream(streams[j]):
                f, x, blob = layers[j]
                outs[j] = ditq.linear(x, blob, 2048, f, ditq.EPI_GATED_SILU)
        torch.cuda.synchronize()
        for j in (0, 1):
            got = outs[j].view(torch.int16).cpu().numpy()
            want = alone[j].view(torch.int16).cpu().numpy()
            assert np.array_equal(got, want), f"repetition {rep}: layer {j} ({(fmt_a, fmt_b)[j]}) differs"
