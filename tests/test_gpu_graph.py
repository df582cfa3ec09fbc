"""The hot path under HIP graph capture (a serving loop replays one captured step).

Quantize + fused GEMM are captured once into a graph on static buffers and
replayed several times, with eager work and synchronisations between the
replays and new activations copied into the static input before some of them.
Every replay must equal the eager result on the same input bit for bit (the
path is deterministic).  NVFP4 is included: its quantizer's three launches
(per-workgroup maxima, their reduction into the tensor-maximum slot, the
quantizer) must all be replayed, or a stale maximum would change the scales.
"""
import numpy as np
import pytest

from workloads import make_inputs

pytestmark = pytest.mark.gpu

FMT = {"fp4": 1, "fp8": 2, "mx8": 3, "nv4": 4}
EPI = {"identity": 0, "gated_silu": 1, "gelu_tanh": 3}


@pytest.fixture(scope="module")
def ditq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_dit_amd
    return bit_gemm_dit_amd


# K = 768 (6 k-steps) selects the FP4 kernels with three fragment buffers, K = 512 the others
@pytest.mark.parametrize("fmt,epi,M,K", [("fp4", "gated_silu", 300, 512), ("fp4", "gated_silu", 300, 768),
                                         ("nv4", "gated_silu", 200, 512), ("mx8", "gelu_tanh", 129, 512),
                                         ("fp8", "identity", 257, 512)])
def test_captured_step_replays_equal_eager(ditq, fmt, epi, M, K):
    import torch
    from tests.gpu_util import to_dev_bf16
    f, e = FMT[fmt], EPI[epi]
    N = 1024
    d0 = make_inputs("mlp_gated_silu", seed=1, M=M, N=N, K=K)
    d1 = make_inputs("mlp_gated_silu", seed=2, M=M, N=N, K=K)
    blob = ditq.pack_weights(to_dev_bf16(d0["w"]), f, e)
    x_static = to_dev_bf16(d0["x"]).clone()
    x_new = to_dev_bf16(d1["x"])

    def step(x):
        codes, scales = ditq.quantize_act(x, f)
        return ditq.gemm(codes, scales, blob, N, K, f, e)

    # eager results for both inputs (also warms up the device check before capture)
    ref0 = step(x_static).clone()
    x_static.copy_(x_new)
    ref1 = step(x_static).clone()
    x_static.copy_(to_dev_bf16(d0["x"]))
    torch.cuda.synchronize()

    print(f"graph capture {fmt} {epi} M={M} K={K}", flush=True)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(x_static)                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        out_static = step(x_static)
    torch.cuda.synchronize()

    for r, (src, ref) in enumerate([(d0, ref0), (d0, ref0), (d1, ref1), (d0, ref0), (d1, ref1)]):
        x_static.copy_(to_dev_bf16(src["x"]))
        step(to_dev_bf16(src["x"]))          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out_static.view(torch.int16).cpu().numpy()
        want = ref.view(torch.int16).cpu().numpy()
        assert np.array_equal(got, want), f"replay {r} differs from the eager result"
