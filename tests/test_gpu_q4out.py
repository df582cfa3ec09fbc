"""GPU parity of the FP4 GEMM whose epilogue also quantizes its output for the next
GEMM (dit_gemm_q4_epilogue_q4).

The quantized output is defined on the bf16 output: it must equal the oracle FP4
quantizer applied to the GPU's bf16 output, bit for bit (codes and scales), and
the bf16 output itself must equal what dit_gemm_q4_epilogue writes, bit for bit,
and lie within the usual tolerance of the float64 oracle.  The codes must also
serve directly as the next GEMM's activations.
"""
import numpy as np
import pytest

from oracle import layer, quant
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

EPI = {"identity": 0, "gated_silu": 1, "qk_rmsnorm": 2, "gelu_tanh": 3}


@pytest.fixture(scope="module")
def ditq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_dit_amd
    return bit_gemm_dit_amd


class Layer:
    """Packed weights and quantized activations of one problem, on the device."""

    def __init__(self, ditq, d, epi):
        import torch
        from tests.gpu_util import to_dev_bf16
        self.d, self.e = d, EPI[epi]
        self.M, self.K = d["x"].shape
        self.N = d["w"].shape[0]
        self.width = self.N // 2 if self.e == 1 else self.N
        self.x = to_dev_bf16(d["x"])
        self.blob = ditq.pack_weights(to_dev_bf16(d["w"]), 1, self.e)
        self.codes, self.scales = ditq.quantize_act(self.x, 1)
        self.keep, self.rms = [], None
        if self.e == 2:
            gq = torch.from_numpy(d["gamma_q"]).cuda()
            gk = torch.from_numpy(d["gamma_k"]).cuda()
            self.keep = [gq, gk]
            self.rms = ditq.rmsnorm_params(gq, gk, d["n_heads"], d["eps"])


def plain_output(ditq, L):
    from tests.gpu_util import to_host_bits
    out = ditq.gemm(L.codes, L.scales, L.blob, L.N, L.K, 1, L.e, rms=L.rms)
    return to_host_bits(out)


def quantized_output(ditq, L, with_bf16):
    import torch
    from tests.gpu_util import to_host_bits
    r = ditq.gemm_q4out(L.codes, L.scales, L.blob, L.N, L.K, L.e, rms=L.rms, with_bf16=with_bf16)
    torch.cuda.synchronize()
    qc, qs = r[0].cpu().numpy(), r[1].cpu().numpy()
    return (qc, qs, to_host_bits(r[2])) if with_bf16 else (qc, qs)


def oracle_rows(d, epi, rows=None):
    kw = {}
    if epi == "qk_rmsnorm":
        kw = dict(n_heads=d["n_heads"], head_dim=d["head_dim"], gamma_q=d["gamma_q"], gamma_k=d["gamma_k"],
                  eps=d["eps"])
    return layer.forward(d["x"], d["w"], "fp4", epi, rows=rows, **kw)


def check_quantized(qc, qs, out_bits, M, width, rows=None):
    """Codes / scales (panel-major) == oracle FP4 quantizer on the bf16 output rows."""
    from tests.gpu_util import act_codes_to_rowmajor, act_scales_to_rowmajor
    codes = act_codes_to_rowmajor(qc, M, width, 1)
    scales = act_scales_to_rowmajor(qs, M, width)
    sel = np.arange(M) if rows is None else np.asarray(rows)
    ref_c, ref_s = quant.quantize_fp4(out_bits[sel] if rows is None else out_bits)
    np.testing.assert_array_equal(scales[sel], ref_s, err_msg="E8M0 scales differ")
    np.testing.assert_array_equal(codes[sel], ref_c, err_msg="E2M1 codes differ")


SMALL = [
    # workload kind, epi, M, N, K, n_heads
    ("tiny_gated_silu", "gated_silu", 130, 512, 256, None),
    ("mlp_gated_silu", "gated_silu", 200, 1024, 3072, None),       # k-steps in groups of 4
    ("mlp_gated_silu", "identity", 70, 512, 512, None),
    ("mlp_gated_silu", "identity", 1, 768, 256, None),
    ("qkv_rmsnorm_hd128", "qk_rmsnorm", 257, None, 256, 2),
    ("qkv_rmsnorm_hd256", "qk_rmsnorm", 65, None, 512, 1),
    ("mlp_gelu_tanh", "gelu_tanh", 130, 768, 512, None),
]


@pytest.mark.parametrize("kind,epi,M,N,K,H", SMALL, ids=[f"{s[1]}-M{s[2]}-K{s[4]}" for s in SMALL])
def test_quantized_output_is_the_quantized_bf16_output(ditq, kind, epi, M, N, K, H):
    from tests.gpu_util import compare_bf16
    d = make_inputs(kind, seed=M + K + 7, M=M, N=N, K=K, n_heads=H)
    print(f"case q4out {kind} {epi} M={M} N={d['w'].shape[0]} K={K}", flush=True)
    L = Layer(ditq, d, epi)
    plain = plain_output(ditq, L)
    qc, qs, out = quantized_output(ditq, L, with_bf16=True)
    np.testing.assert_array_equal(out, plain, err_msg="bf16 output differs from dit_gemm_q4_epilogue")
    check_quantized(qc, qs, out, L.M, L.width)
    qc2, qs2 = quantized_output(ditq, L, with_bf16=False)
    np.testing.assert_array_equal(qc2, qc)
    np.testing.assert_array_equal(qs2, qs)
    compare_bf16(out, oracle_rows(d, epi), f"{kind}/{epi}")


def test_quantized_output_feeds_the_next_gemm(ditq):
    """Layer 1 (gated-SiLU, quantized output) -> layer 2 (identity): the same result
    as quantizing layer 1's bf16 output with dit_quantize_act."""
    import torch
    from tests.gpu_util import to_dev_bf16, to_host_bits
    d1 = make_inputs("mlp_gated_silu", seed=11, M=300, N=1024, K=512)
    L1 = Layer(ditq, d1, "gated_silu")
    qc, qs, out = ditq.gemm_q4out(L1.codes, L1.scales, L1.blob, L1.N, L1.K, L1.e, with_bf16=True)
    ref_c, ref_s = ditq.quantize_act(out, 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(qc.cpu().numpy(), ref_c.cpu().numpy())
    np.testing.assert_array_equal(qs.cpu().numpy(), ref_s.cpu().numpy())
    d2 = make_inputs("mlp_gated_silu", seed=12, M=300, N=768, K=512)
    blob2 = ditq.pack_weights(to_dev_bf16(d2["w"]), 1, 0)
    y_fused = ditq.gemm(qc, qs, blob2, 768, 512, 1, 0)
    y_ref = ditq.gemm(ref_c, ref_s, blob2, 768, 512, 1, 0)
    np.testing.assert_array_equal(to_host_bits(y_fused), to_host_bits(y_ref))


def test_full_size_headline_every_element(ditq):
    """The headline workload in the benchmark's launch configuration: every code and
    scale byte, and every bf16 element against the oracle."""
    from tests.gpu_util import compare_bf16
    d = make_inputs("mlp_gated_silu", seed=0)
    print("case q4out full mlp_gated_silu", flush=True)
    L = Layer(ditq, d, "gated_silu")
    qc, qs, out = quantized_output(ditq, L, with_bf16=True)
    check_quantized(qc, qs, out, L.M, L.width)
    compare_bf16(out, oracle_rows(d, "gated_silu"), "q4out full")
