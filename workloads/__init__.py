"""Seeded synthetic inputs for the fused low-bit DiT linear layer.

This module is shared by the tests, the benchmark and the CPU oracle's tests.
It holds no arithmetic of the method itself: it only draws random tensors with
the shapes and value distributions of the workloads and rounds them to bf16,
the input type of the layer.

Workloads (shapes are GEMM M x N x K, N = full GEMM width):

* ``tiny_gated_silu``   64 x 512 x 256, FP4, gated-SiLU, no outliers.
* ``qkv_rmsnorm_hd128`` 4608 x 9216 x 3072, FP4, per-head QK-RMSNorm, 24 heads of 128.
  4608 tokens = 4096 image tokens (1024^2 image -> 128^2 latent, patch 2) + 512 text tokens.
* ``mlp_gated_silu``    4608 x 16384 x 3072, FP4, gated-SiLU over 8192 gate/up pairs.
* ``qkv_rmsnorm_hd256`` 4096 x 12288 x 4096, FP4, per-head QK-RMSNorm, 16 heads of 256.
* ``fp8_cfg_pair``      9216 x 12288 x 3072, FP8 E4M3, identity and gated-SiLU;
  9216 = 2 x 4608 tokens (the conditional and unconditional halves of a CFG pair).
* ``mlp_gelu_tanh``     4608 x 12288 x 3072, FP4, GELU (tanh form): a FLUX-style
  MLP up-projection (hidden 3072, ratio 4).
* ``mlp_down_gate_residual`` 9216 x 3072 x 12288, FP4, gated residual update: the
  MLP down-projection of a CFG pair, out = residual + gate[sample] * C, one gate
  row per sample of 4608 tokens.

Value distributions: activations ~ N(0, 1) with 1 % of the K channels (the same
channels for every row) scaled by 20; weights ~ N(0, 1/sqrt(K)) (standard
deviation 1/sqrt(K)); RMSNorm gammas ~ U(0.5, 1.5); eps = 1e-6; residual ~ N(0, 1)
(bf16, [M, N]); gates ~ N(0, 0.5^2) (fp32, one row of N per sample).

The diffusion-transformer shapes follow the DiT layers the pages accelerate
(FLUX-dev: hidden 3072, 24 heads of 128; page "WaveSpeedAI X DataCrunch: FLUX
real-time image inference on B200", section on FLUX-dev) and the epilogues of
page "How fal made Ideogram V4 6x faster" (news.ditty.ir), paragraphs on epilogue
fusion and gated-SiLU.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

FP4 = "fp4"
FP8 = "fp8"
IDENTITY = "identity"
GATED_SILU = "gated_silu"
QK_RMSNORM = "qk_rmsnorm"
GELU_TANH = "gelu_tanh"
GATE_RESIDUAL = "gate_residual"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    fmt: str
    epis: tuple
    M: int
    N: int
    K: int
    outliers: bool
    n_heads: int = 0
    head_dim: int = 0
    eps: float = 1e-6
    rows_per_gate: int = 0       # tokens per sample of the gated residual (0: no gate)

    @property
    def flops(self) -> int:
        """2*M*N*K with N the full GEMM width (gate and up columns both counted)."""
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    "tiny_gated_silu": Workload("tiny_gated_silu", FP4, (GATED_SILU,), 64, 512, 256, False),
    "qkv_rmsnorm_hd128": Workload("qkv_rmsnorm_hd128", FP4, (QK_RMSNORM,), 4608, 9216, 3072, True,
                                  n_heads=24, head_dim=128),
    "mlp_gated_silu": Workload("mlp_gated_silu", FP4, (GATED_SILU,), 4608, 16384, 3072, True),
    "qkv_rmsnorm_hd256": Workload("qkv_rmsnorm_hd256", FP4, (QK_RMSNORM,), 4096, 12288, 4096, True,
                                  n_heads=16, head_dim=256),
    "fp8_cfg_pair": Workload("fp8_cfg_pair", FP8, (IDENTITY, GATED_SILU), 9216, 12288, 3072, True),
    "mlp_gelu_tanh": Workload("mlp_gelu_tanh", FP4, (GELU_TANH,), 4608, 12288, 3072, True),
    "mlp_down_gate_residual": Workload("mlp_down_gate_residual", FP4, (GATE_RESIDUAL,), 9216, 3072, 12288, True,
                                       rows_per_gate=4608),
}
ORDER = ["tiny_gated_silu", "qkv_rmsnorm_hd128", "mlp_gated_silu", "qkv_rmsnorm_hd256", "fp8_cfg_pair",
         "mlp_gelu_tanh", "mlp_down_gate_residual"]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns.

    Inputs are finite by construction here, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(rng: np.random.Generator, K: int) -> np.ndarray:
    return rng.choice(K, int(round(0.01 * K)), replace=False)


def make_inputs(wl: Workload | str, seed: int = 0, M: int | None = None, N: int | None = None,
                K: int | None = None, n_heads: int | None = None, rows_per_gate: int | None = None) -> dict:
    """Draw the inputs of one workload.

    Draw order (one PCG64 generator per call): outlier channel indices, the
    activation matrix [M, K], the weight matrix [N, K] (rows in gate-then-up
    order for gated-SiLU), then gamma_q and gamma_k, then (gated residual) the
    residual [M, N] and the gates [ceil(M / rows_per_gate), N].  M, N, K,
    n_heads and rows_per_gate may be overridden to get smaller problems of the
    same kind for parity tests.

    Returns a dict with ``x`` (uint16 bf16 bits [M, K]), ``w`` (uint16 bf16 bits
    [N, K]), ``gamma_q`` / ``gamma_k`` (float32 [head_dim] or None), ``eps``,
    ``residual`` (uint16 bf16 bits [M, N] or None), ``gate`` (float32 or None),
    ``rows_per_gate``.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    M = wl.M if M is None else M
    K = wl.K if K is None else K
    H = wl.n_heads if n_heads is None else n_heads
    if N is None:
        N = wl.N if n_heads is None else 3 * H * wl.head_dim
    rng = np.random.default_rng(seed)
    chans = outlier_channels(rng, K) if wl.outliers else np.zeros(0, dtype=np.int64)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if chans.size:
        x[:, chans] *= np.float32(20.0)
    w = rng.standard_normal((N, K), dtype=np.float32) / np.float32(math.sqrt(K))
    gq = gk = None
    if wl.head_dim:
        gq = rng.uniform(0.5, 1.5, wl.head_dim).astype(np.float32)
        gk = rng.uniform(0.5, 1.5, wl.head_dim).astype(np.float32)
    rpg = wl.rows_per_gate if rows_per_gate is None else rows_per_gate
    res = gate = None
    if rpg:
        res = f32_to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32))
        gate = (rng.standard_normal(((M + rpg - 1) // rpg, N), dtype=np.float32) * np.float32(0.5))
    return {
        "x": f32_to_bf16_bits(x),
        "w": f32_to_bf16_bits(w),
        "gamma_q": gq,
        "gamma_k": gk,
        "eps": wl.eps,
        "outlier_channels": chans,
        "residual": res,
        "gate": gate,
        "rows_per_gate": rpg,
        "M": M, "N": N, "K": K, "n_heads": H, "head_dim": wl.head_dim,
    }
