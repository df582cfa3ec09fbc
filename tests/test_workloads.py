"""The seeded input generator: shapes, determinism and the outlier recipe."""
import numpy as np

from workloads import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -9, -2.5], dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 1.5*2^-8 -> 1 + 2^-7
    np.testing.assert_array_equal(bf16_bits_to_f32(f32_to_bf16_bits(x)), [1.0, 1.0, 1.0078125, 1.0078125, -2.5])


def test_tiny_workload_shapes_and_seed():
    a = make_inputs("tiny_gated_silu", seed=0)
    b = make_inputs("tiny_gated_silu", seed=0)
    assert a["x"].shape == (64, 256) and a["w"].shape == (512, 256)
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["w"], b["w"])
    assert a["outlier_channels"].size == 0


def test_outliers_and_overrides():
    d = make_inputs("qkv_rmsnorm_hd128", seed=0, M=40, n_heads=2)
    assert d["x"].shape == (40, 3072) and d["w"].shape == (3 * 2 * 128, 3072)
    ch = d["outlier_channels"]
    assert ch.size == 31 and len(set(ch.tolist())) == 31
    x = bf16_bits_to_f32(d["x"])
    assert np.abs(x[:, ch]).mean() > 10 * np.abs(np.delete(x, ch, axis=1)).mean()
    assert d["gamma_q"].shape == (128,) and 0.5 <= d["gamma_q"].min() and d["gamma_k"].max() <= 1.5


def test_workload_table():
    assert WORKLOADS["mlp_gated_silu"].flops == 2 * 4608 * 16384 * 3072
    assert WORKLOADS["qkv_rmsnorm_hd256"].N == 3 * 16 * 256
    assert WORKLOADS["qkv_rmsnorm_hd128"].N == 3 * 24 * 128


def test_gate_residual_inputs():
    d = make_inputs("mlp_down_gate_residual", seed=1, M=50, N=128, K=256, rows_per_gate=20)
    assert d["residual"].shape == (50, 128) and d["gate"].shape == (3, 128) and d["rows_per_gate"] == 20
    assert d["gate"].dtype == np.float32 and 0.3 < float(np.std(d["gate"])) < 0.7
    e = make_inputs("mlp_gated_silu", seed=1, M=8, N=128, K=256)
    assert e["residual"] is None and e["gate"] is None
    assert WORKLOADS["mlp_down_gate_residual"].flops == 2 * 9216 * 3072 * 12288
