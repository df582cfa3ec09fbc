"""GPU parity of the split-last-round GEMMs (dit_gemm_epilogue_ws,
dit_gemm_gate_residual_ws) against the float64 oracle.

With a work space, the tiles of a partly empty last round are split along K over
the idle compute units and their fp32 parts summed before the epilogue.  The
result must meet the same per-element tolerance as the unsplit call (it sums the
same products in another grouping).  Small shapes have fewer tiles than CUs, so
every tile is split (up to 8 ways); the full-size shapes split only their last
round.  Also checked: the work space's flags are zero again after every call and no
flag wait gave up; two calls give identical bits; a captured graph replays
correctly; two streams with their own work spaces run at once.
"""
import numpy as np
import pytest

from tests.test_gpu_gemm import EPI, FMT, oracle_rows
from workloads import make_inputs

pytestmark = pytest.mark.gpu

FLAG_BYTES = 32 * 1024           # the flag area at the start of the work space (and the give-up count)


@pytest.fixture(scope="module")
def ditq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_dit_amd
    return bit_gemm_dit_amd


@pytest.fixture(scope="module")
def ws(ditq):
    return ditq.gemm_workspace()


def prepare(ditq, d, fmt, epi):
    """Packed weights, quantized activations and the RMSNorm / gated-residual
    parameters of one problem (device tensors kept in the returned dict)."""
    import torch
    from tests.gpu_util import to_dev_bf16
    M, K = d["x"].shape
    N = d["w"].shape[0]
    f, e = FMT[fmt], EPI[epi]
    st = torch.cuda.current_stream().cuda_stream
    x, w = to_dev_bf16(d["x"]), to_dev_bf16(d["w"])
    blob = torch.empty(ditq.dit_packed_weight_bytes(f, e, N, K), dtype=torch.uint8, device="cuda")
    ditq.dit_pack_weights(f, e, w.data_ptr(), N, K, K, blob.data_ptr(), st)
    codes = torch.empty(ditq.dit_act_code_bytes(f, M, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty(ditq.dit_act_scale_bytes(f, M, K), dtype=torch.uint8, device="cuda")
    ditq.dit_quantize_act(f, x.data_ptr(), M, K, K, codes.data_ptr(), scales.data_ptr(), st)
    p = dict(M=M, N=N, K=K, f=f, e=e, blob=blob, codes=codes, scales=scales, rms=None, gr=None,
             width=N // 2 if e == 1 else N)
    if e == 2:
        p["gq"], p["gk"] = torch.from_numpy(d["gamma_q"]).cuda(), torch.from_numpy(d["gamma_k"]).cuda()
        p["rms"] = ditq.RmsNormParams(d["head_dim"], d["n_heads"], p["gq"].data_ptr(), p["gk"].data_ptr(), d["eps"])
    if e == 4:
        p["res"], p["gate"] = to_dev_bf16(d["residual"]), torch.from_numpy(d["gate"]).cuda()
        p["gr"] = ditq.GateResidualParams(p["res"].data_ptr(), N, p["gate"].data_ptr(), d["rows_per_gate"])
    return p


def launch(ditq, p, out, ws, stream):
    """One split call into `out` (int16 device tensor [M, width]) on `stream` (a raw handle)."""
    nbytes = ws.numel() if ws is not None else 0
    wptr = ws.data_ptr() if ws is not None else None
    if p["e"] == 4:
        ditq.dit_gemm_gate_residual_ws(p["f"], p["codes"].data_ptr(), p["scales"].data_ptr(), p["blob"].data_ptr(),
                                       p["M"], p["N"], p["K"], p["gr"], out.data_ptr(), p["width"], wptr, nbytes,
                                       stream)
    else:
        ditq.dit_gemm_epilogue_ws(p["f"], p["codes"].data_ptr(), p["scales"].data_ptr(), p["blob"].data_ptr(),
                                  p["M"], p["N"], p["K"], p["e"], p["rms"], out.data_ptr(), p["width"], wptr, nbytes,
                                  stream)


def run(ditq, p, ws):
    import torch
    out = torch.full((p["M"], p["width"]), -12345, dtype=torch.int16, device="cuda")
    launch(ditq, p, out, ws, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def assert_workspace_clean(ws):
    flags = ws[:FLAG_BYTES].cpu().numpy()
    assert not flags.any(), f"work space flags left set ({int(np.count_nonzero(flags))} bytes)"


def case_inputs(kind, M, N, K, H):
    if H is None:
        return make_inputs(kind, seed=3, M=M, N=N, K=K)
    return make_inputs(kind, seed=3, M=M, K=K, n_heads=H)


SMALL = [
    # workload kind, fmt, epi, M, N, K, n_heads: fewer tiles than CUs, so every tile is split
    ("mlp_gated_silu", "fp4", "gated_silu", 300, 1024, 3072, None),
    ("mlp_gated_silu", "fp4", "identity", 257, 832, 1024, None),
    ("mlp_gated_silu", "fp4", "gated_silu", 1, 640, 768, None),
    ("qkv_rmsnorm_hd128", "fp4", "qk_rmsnorm", 300, None, 1024, 2),
    ("qkv_rmsnorm_hd256", "fp4", "qk_rmsnorm", 130, None, 2048, 1),
    ("mlp_gelu_tanh", "fp4", "gelu_tanh", 300, 768, 1536, None),
    ("fp8_cfg_pair", "fp8", "identity", 300, 768, 2048, None),
    ("fp8_cfg_pair", "fp8", "gated_silu", 129, 1024, 768, None),
    ("qkv_rmsnorm_hd128", "fp8", "qk_rmsnorm", 300, None, 1024, 2),
    ("mlp_gated_silu", "mx8", "gated_silu", 200, 1024, 2048, None),
    ("qkv_rmsnorm_hd256", "mx8", "qk_rmsnorm", 65, None, 1024, 1),
    ("mlp_gated_silu", "nv4", "gated_silu", 300, 1024, 1024, None),
    ("qkv_rmsnorm_hd128", "nv4", "qk_rmsnorm", 257, None, 512, 2),
    ("mlp_gelu_tanh", "mx8", "gelu_tanh", 70, 1024, 1152, None),
]


@pytest.mark.parametrize("kind,fmt,epi,M,N,K,H", SMALL, ids=[f"{s[1]}-{s[2]}-M{s[3]}-K{s[5]}" for s in SMALL])
def test_small_split_all_elements(ditq, ws, kind, fmt, epi, M, N, K, H):
    from tests.gpu_util import compare_bf16
    print(f"case split small {fmt} {epi} M={M} K={K}", flush=True)
    d = case_inputs(kind, M, N, K, H)
    p = prepare(ditq, d, fmt, epi)
    g = run(ditq, p, ws)
    assert_workspace_clean(ws)
    compare_bf16(g, oracle_rows(d, fmt, epi), f"split {fmt}/{epi} M={M} K={K}")


GR = [("fp4", 300, 512, 2048, 100), ("fp8", 257, 512, 768, 129), ("mx8", 200, 768, 1024, 64),
      ("nv4", 130, 512, 512, 50)]


@pytest.mark.parametrize("fmt,M,N,K,rpg", GR, ids=[f"{g[0]}-M{g[1]}-K{g[3]}" for g in GR])
def test_gate_residual_split_all_elements(ditq, ws, fmt, M, N, K, rpg):
    from tests.gpu_util import compare_bf16
    print(f"case split gated residual {fmt} M={M} K={K}", flush=True)
    d = make_inputs("mlp_down_gate_residual", seed=5, M=M, N=N, K=K, rows_per_gate=rpg)
    p = prepare(ditq, d, fmt, "gate_residual")
    g = run(ditq, p, ws)
    assert_workspace_clean(ws)
    compare_bf16(g, oracle_rows(d, fmt, "gate_residual"), f"split gated residual {fmt}")


FULL = [("qkv_rmsnorm_hd128", "qk_rmsnorm", "fp4"), ("mlp_gelu_tanh", "gelu_tanh", "fp4"),
        ("mlp_down_gate_residual", "gate_residual", "fp4"), ("qkv_rmsnorm_hd256", "qk_rmsnorm", "fp8"),
        ("qkv_rmsnorm_hd128", "qk_rmsnorm", "fp8"), ("mlp_gated_silu", "gated_silu", "fp4")]


@pytest.mark.parametrize("name,epi,fmt", FULL, ids=[f"{a}-{b}-{c}" for a, b, c in FULL])
def test_full_size_split_every_element(ditq, ws, name, epi, fmt):
    """The full-size shapes whose last round is partly empty (and the headline, which
    fills whole rounds and so runs the plain kernel): every element."""
    from tests.gpu_util import compare_bf16
    print(f"case split full {name} {epi} {fmt}", flush=True)
    d = make_inputs(name, seed=0)
    p = prepare(ditq, d, fmt, epi)
    g = run(ditq, p, ws)
    assert_workspace_clean(ws)
    compare_bf16(g, oracle_rows(d, fmt, epi), f"split {name}/{epi}/{fmt}")


def test_deterministic_and_graph_replay(ditq, ws):
    """Two eager calls give identical bits; a captured split call replayed three times,
    with eager work and new inputs in between, matches the eager result each time."""
    import torch
    print("case split determinism + graph", flush=True)
    d = make_inputs("qkv_rmsnorm_hd128", seed=9, M=300, K=1024, n_heads=2)
    p = prepare(ditq, d, "fp4", "qk_rmsnorm")
    a, b = run(ditq, p, ws), run(ditq, p, ws)
    np.testing.assert_array_equal(a, b)
    s = torch.cuda.Stream()
    out = torch.zeros((p["M"], p["width"]), dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        launch(ditq, p, out, ws, s.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(-1)
        junk = torch.randn(1 << 20, device="cuda").sum()        # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), a, err_msg=f"replay {rep}")
        assert_workspace_clean(ws)
        del junk


def test_two_streams_own_work_spaces(ditq, ws):
    """Two split calls on two streams at once, each with its own work space: each result
    equals the same call alone, bit for bit, and both work spaces end clean."""
    import torch
    print("case split two streams", flush=True)
    d1 = make_inputs("mlp_gelu_tanh", seed=11, M=300, N=768, K=1536)
    d2 = make_inputs("qkv_rmsnorm_hd128", seed=12, M=257, K=1024, n_heads=2)
    p1, p2 = prepare(ditq, d1, "fp4", "gelu_tanh"), prepare(ditq, d2, "fp4", "qk_rmsnorm")
    ref1, ref2 = run(ditq, p1, ws), run(ditq, p2, ws)
    ws2 = ditq.gemm_workspace()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        o1 = torch.zeros((p1["M"], p1["width"]), dtype=torch.int16, device="cuda")
        o2 = torch.zeros((p2["M"], p2["width"]), dtype=torch.int16, device="cuda")
        torch.cuda.synchronize()
        launch(ditq, p1, o1, ws, s1.cuda_stream)
        launch(ditq, p2, o2, ws2, s2.cuda_stream)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(o1.cpu().numpy().view(np.uint16), ref1)
        np.testing.assert_array_equal(o2.cpu().numpy().view(np.uint16), ref2)
    assert_workspace_clean(ws)
    assert_workspace_clean(ws2)


def test_null_work_space_is_the_plain_call(ditq):
    """workspace NULL: the entry point without _ws, bit for bit."""
    import torch
    d = make_inputs("mlp_gelu_tanh", seed=13, M=300, N=768, K=1536)
    p = prepare(ditq, d, "fp4", "gelu_tanh")
    g = run(ditq, p, None)
    out = torch.full((p["M"], p["width"]), -12345, dtype=torch.int16, device="cuda")
    ditq.dit_gemm_epilogue(p["f"], p["codes"].data_ptr(), p["scales"].data_ptr(), p["blob"].data_ptr(), p["M"], p["N"],
                           p["K"], p["e"], None, out.data_ptr(), p["width"], torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(g, out.cpu().numpy().view(np.uint16))
