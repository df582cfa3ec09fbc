"""bench.py's contract, checked without a GPU: the multi-GPU refusal, and the
traffic figure that is reported only while the profile describes the current kernel
source."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "WORLD_SIZE": "1"})
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    assert len(h) == 16
    good = tmp_path / "traffic.txt"
    good.write_text(f"# comment\nsource_hash={h}\nhbm_bytes_per_launch=279000000\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.read_traffic() == 279000000.0
    stale = tmp_path / "stale.txt"
    stale.write_text("source_hash=0000000000000000\nhbm_bytes_per_launch=279000000\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.read_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.read_traffic() is None


def test_source_hash_covers_the_gemm_sources(tmp_path, monkeypatch):
    src = tmp_path / "gemm.hip"
    src.write_text(open(bench.GEMM_SRC).read())
    monkeypatch.setattr(bench, "GEMM_SRC", str(src))
    h0 = bench.kernel_source_hash()
    src.write_text(src.read_text() + "\n// a comment only\n")
    assert bench.kernel_source_hash() == h0
    src.write_text(src.read_text() + "\nconstexpr int kChanged = 1;\n")
    assert bench.kernel_source_hash() != h0


def test_oracle_rate_runs_for_every_format_and_epilogue():
    """bench.py --all-configs times the oracle beside each workload; every format and
    epilogue it uses must run on a small problem of the same kind."""
    from workloads import make_inputs
    cases = [("tiny_gated_silu", "fp4", "gated_silu", {}), ("qkv_rmsnorm_hd128", "fp8", "qk_rmsnorm",
             dict(M=64, n_heads=1)), ("mlp_gelu_tanh", "mx8", "gelu_tanh", dict(M=64, N=256, K=256)),
             ("mlp_down_gate_residual", "fp4", "gate_residual", dict(M=64, N=256, K=256, rows_per_gate=32)),
             ("tiny_gated_silu", "nv4", "identity", {})]
    for name, fmt, epi, kw in cases:
        d = make_inputs(name, seed=1, **kw)
        r = bench.oracle_rate(d, fmt, epi, 0.05)
        assert r["value"] > 0 and r["kind"] == "oracle" and r["unit"] == "TFLOP/s", (name, fmt, epi, r)


def test_kernel_hash_ignores_comments_only():
    """The counter summaries stay valid across comment edits, not across code edits."""
    import bench
    src = "int a = 1;  // one\n/* block\n comment */\nint b = 2;\n\n// trailing\n"
    assert bench.code_only(src) == "int a = 1;\nint b = 2;"
    assert bench.code_only(src.replace("// one", "// first")) == bench.code_only(src)
    assert bench.code_only(src.replace("b = 2", "b = 3")) != bench.code_only(src)
