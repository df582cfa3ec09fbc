"""Seeded random shapes through every format and epilogue (GPU parity against the oracle).

Each case is drawn from one seeded generator:
- a format (FP4, FP8 row/column, MXFP8, NVFP4);
- an epilogue (identity, gated-SiLU, GELU-tanh, QK-RMSNorm with head_dim 128 or
  256, gated residual);
- M in [1, 700] and K a multiple of 256 up to 1536;
- N a multiple of 64 (of 128 for gated-SiLU; 3 x heads x head_dim for QK-RMSNorm);
- an output row stride with up to 24 elements of padding;
- for the gated residual, the rows per gate.

Every element is compared with the oracle, guard bytes around the output and its
padding must stay untouched, and the residual must only be read.  The fixed cases
of test_gpu_gemm.py pin chosen shapes; these cover the combinations in between.
The environment variables DITQ_FUZZ_CASES and DITQ_FUZZ_SEED set a longer or another list
for a soak run.
"""
import os

import numpy as np
import pytest

from tests.test_gpu_gemm import oracle_rows, run_gate_residual, run_layer

pytestmark = pytest.mark.gpu

KIND = {"identity": "mlp_gated_silu", "gated_silu": "mlp_gated_silu", "gelu_tanh": "mlp_gelu_tanh",
        "rms128": "qkv_rmsnorm_hd128", "rms256": "qkv_rmsnorm_hd256", "gate_residual": "mlp_down_gate_residual"}


def _cases(n=200, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = ["fp4", "fp8", "mx8", "nv4"][i % 4]
        epi = ["identity", "gated_silu", "gelu_tanh", "rms128", "rms256", "gate_residual"][rng.integers(0, 6)]
        M = int(rng.choice([1, 2, 31, 33, 191, 193, 257]) if rng.random() < 0.4 else rng.integers(1, 701))
        K = int(256 * rng.integers(1, 7))
        H = None
        rpg = None
        if epi == "gated_silu":
            N = int(128 * rng.integers(1, 17))
        elif epi == "rms128":
            H = int(rng.integers(1, 5))
            N = 3 * 128 * H
        elif epi == "rms256":
            H = int(rng.integers(1, 3))
            N = 3 * 256 * H
        else:
            N = int(64 * rng.integers(1, 26))
        if epi == "gate_residual":
            rpg = int(rng.integers(1, M + 1))
        pad = int(8 * rng.integers(0, 4))
        out.append((i, fmt, epi, M, N, K, H, rpg, pad))
    return out


# DITQ_FUZZ_CASES draws a longer list (the first 200 cases are always the same);
# DITQ_FUZZ_SEED draws another list
CASES = _cases(int(os.environ.get("DITQ_FUZZ_CASES", "200")), int(os.environ.get("DITQ_FUZZ_SEED", "2024")))


@pytest.fixture(scope="module")
def ditq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_dit_amd
    return bit_gemm_dit_amd


@pytest.mark.parametrize("i,fmt,epi,M,N,K,H,rpg,pad", CASES,
                         ids=[f"{c[0]}-{c[1]}-{c[2]}-M{c[3]}-N{c[4]}-K{c[5]}" for c in CASES])
def test_random_shape(ditq, i, fmt, epi, M, N, K, H, rpg, pad):
    from tests.gpu_util import compare_bf16
    from workloads import make_inputs
    d = make_inputs(KIND[epi], seed=1000 + i, M=M, N=None if H else N, K=K, n_heads=H, rows_per_gate=rpg)
    N = d["w"].shape[0]
    print(f"fuzz case {i}: {fmt} {epi} M={M} N={N} K={K} heads={H} rows_per_gate={rpg} pad={pad}", flush=True)
    if epi == "gate_residual":
        g = run_gate_residual(ditq, d, fmt, ldo=N + pad, guard=32)
        y = oracle_rows(d, fmt, "gate_residual")
    else:
        e = "qk_rmsnorm" if epi.startswith("rms") else epi
        width = N // 2 if e == "gated_silu" else N
        g = run_layer(ditq, d, fmt, e, ldo=width + pad, guard=32)
        y = oracle_rows(d, fmt, e)
    compare_bf16(g, y, f"fuzz {i} {fmt}/{epi}")
