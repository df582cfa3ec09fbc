"""The C ABI on the CPU: the library loads, exports every function include/*.h
declares, its size queries are right, and every validation path returns its
status before any HIP call (fake pointers are never dereferenced)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

ditq = pytest.importorskip("bit_gemm_dit_amd", reason="libditq.so not built")

OK, EINVAL, EUNSUP, EALIGN, EDEVICE = 0, 1, 2, 3, 4
A = 0x10000          # fake, 16-byte aligned "device" addresses: never dereferenced
B = 0x20000
C = 0x30000
D = 0x40000


def _declared():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(dit_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = _declared()
    assert names == sorted(ditq.EXPORTED)
    lib = ctypes.CDLL(ditq.library_path)
    for n in names:
        assert hasattr(lib, n), n


def test_size_queries():
    assert ditq.dit_act_code_bytes(1, 4608, 3072) == 4608 * 1536
    assert ditq.dit_act_scale_bytes(1, 4608, 3072) == 4608 * 96
    assert ditq.dit_act_code_bytes(2, 9216, 3072) == 9216 * 3072
    assert ditq.dit_act_scale_bytes(2, 9216, 3072) == 9216 * 4
    assert ditq.dit_packed_weight_bytes(1, 1, 16384, 3072) == 256 + 16384 * 1536 + 16384 * 96
    assert ditq.dit_packed_weight_bytes(1, 0, 320, 256) == 256 + 512 * 128 + 512 * 8     # rows padded to 512
    assert ditq.dit_packed_weight_bytes(2, 0, 12288, 3072) == 256 + 12288 * 3072 + 12288 * 4
    assert ditq.dit_packed_weight_bytes(1, 0, 64, 128) == 256 + 256 * 64 + 256 * 4    # K = 128: one k-step
    assert ditq.dit_packed_weight_bytes(1, 0, 64, 384) == 256 + 256 * 192 + 256 * 12  # K = 3 * 128
    assert ditq.dit_packed_weight_bytes(1, 0, 64, 192) == 0          # K % 128
    assert ditq.dit_act_code_bytes(1, 10, 384) == 10 * 192 and ditq.dit_act_code_bytes(1, 10, 320) == 0
    assert ditq.dit_packed_weight_bytes(1, 1, 64, 256) == 0          # gated needs N % 128
    assert ditq.dit_packed_weight_bytes(2, 2, 384, 256) == 256 + 512 * 256 + 512 * 4   # = the identity blob
    assert ditq.dit_packed_weight_bytes(3, 0, 64, 256) == 256 + 256 * 256 + 256 * 8    # MXFP8
    assert ditq.dit_packed_weight_bytes(3, 1, 16384, 3072) == 256 + 16384 * 3072 + 16384 * 96
    assert ditq.dit_act_code_bytes(3, 4608, 3072) == 4608 * 3072
    assert ditq.dit_act_scale_bytes(3, 4608, 3072) == 4608 * 96
    assert ditq.dit_packed_weight_bytes(4, 0, 64, 256) == 256 + 256 * 128 + 256 * 16   # NVFP4
    assert ditq.dit_act_code_bytes(4, 64, 256) == 64 * 128
    assert ditq.dit_act_scale_bytes(4, 64, 256) == 64 * 16 + 16 + 2048   # + the tensor-scale tail and work space
    assert ditq.dit_packed_weight_bytes(5, 0, 64, 256) == 0          # no such format
    assert ditq.dit_act_code_bytes(5, 64, 256) == 0
    assert ditq.dit_act_code_bytes(1, 0, 256) == 0


def test_status_strings():
    for s in range(5):
        assert ditq.dit_status_str(s)
    assert ditq.dit_status_str(99) == "unknown status"


def _q4(a=A, s=B, w=C, M=64, N=512, K=256, epi=1, rms=None, out=D, ldo=256):
    return ditq._lib.dit_gemm_q4_epilogue(a, s, w, M, N, K, epi, ctypes.byref(rms) if rms else None, out, ldo, None)


def test_gemm_q4_validation():
    assert _q4(a=None) == EINVAL
    assert _q4(M=0) == EINVAL
    assert _q4(epi=7) == EINVAL
    assert _q4(epi=2) == EINVAL                                      # RMSNorm without params
    r = ditq.RmsNormParams(128, 1, A, B, 1e-6)
    assert _q4(epi=1, rms=r) == EINVAL                               # params without RMSNorm
    assert _q4(epi=2, rms=r, N=512) == EINVAL                        # N != 3 H D
    assert _q4(epi=2, rms=ditq.RmsNormParams(128, 1, A, B, 0.0), N=384, ldo=384) == EINVAL   # eps <= 0
    assert _q4(epi=2, rms=ditq.RmsNormParams(64, 2, A, B, 1e-6), N=384, ldo=384) == EUNSUP   # head_dim 64
    assert _q4(K=192) == EUNSUP                                      # K % 128
    assert _q4(N=576) == EUNSUP                                      # gated needs N % 128
    assert _q4(out=D + 8) == EALIGN
    assert _q4(ldo=255) == EALIGN                                    # < output width 256
    assert _q4(ldo=260) == EALIGN                                    # not a multiple of 8
    assert _q4(epi=0, ldo=256) == EALIGN                             # identity width is 512
    assert _q4(s=B + 4) == EALIGN
    # every argument valid: the first HIP call reports that no gfx950 device is usable
    if not _has_gpu():
        assert _q4() == EDEVICE
        assert _q4(K=384) == EDEVICE                                 # K = 3 * 128 is accepted
        assert _q4(K=128) == EDEVICE


E = 0x50000
F = 0x60000


def _q4q(a=A, s=B, w=C, M=64, N=512, K=256, epi=1, rms=None, out=D, ldo=256, qc=E, qs=F):
    return ditq._lib.dit_gemm_q4_epilogue_q4(a, s, w, M, N, K, epi, ctypes.byref(rms) if rms else None, out, ldo,
                                             qc, qs, None)


def test_gemm_q4_quantized_output_validation():
    assert _q4q(qc=None) == EINVAL
    assert _q4q(qs=None) == EINVAL
    assert _q4q(a=None) == EINVAL
    assert _q4q(epi=2) == EINVAL                                     # RMSNorm without params
    assert _q4q(N=384) == EUNSUP                                     # gated output width 192: not whole k-steps
    assert _q4q(epi=0, N=320, ldo=320) == EUNSUP                     # identity output width 320
    assert _q4q(qc=E + 4) == EALIGN
    assert _q4q(qs=F + 8) == EALIGN
    assert _q4q(ldo=255) == EALIGN                                   # a bf16 output still needs its ldo
    # the bf16 output is optional: without it ldo is not looked at
    if not _has_gpu():
        assert _q4q(out=None, ldo=0) == EDEVICE
        assert _q4q() == EDEVICE
        assert _q4q(epi=2, rms=ditq.RmsNormParams(128, 2, A, B, 1e-6), N=768, ldo=768) == EDEVICE


def test_other_entry_points_validation():
    lib = ditq._lib
    assert lib.dit_quantize_act(1, None, 4, 256, 256, B, C, None) == EINVAL
    assert lib.dit_quantize_act(5, A, 4, 256, 256, B, C, None) == EINVAL
    assert lib.dit_quantize_act(4, A, 4, 256, 256, B, C + 4, None) == EALIGN       # NVFP4 scales: 16 B
    assert lib.dit_quantize_act(3, A, 4, 256, 256, None, C, None) == EINVAL
    assert lib.dit_quantize_act(3, A, 4, 256, 256, B + 8, C, None) == EALIGN       # MXFP8 codes need 16 B
    assert lib.dit_quantize_act(1, A, 4, 300, 304, B, C, None) == EUNSUP
    assert lib.dit_quantize_act(1, A, 4, 192, 192, B, C, None) == EUNSUP          # K % 128
    assert lib.dit_quantize_act(1, A, 4, 256, 250, B, C, None) == EALIGN
    assert lib.dit_quantize_act(1, A + 2, 4, 256, 256, B, C, None) == EALIGN
    assert lib.dit_quantize_act(2, A, 4, 256, 256, B, C + 2, None) == EALIGN
    assert lib.dit_pack_weights(1, 0, A, 64, 256, 256, None, None) == EINVAL
    assert lib.dit_pack_weights(1, 1, A, 64, 256, 256, B, None) == EUNSUP
    assert lib.dit_pack_weights(3, 1, A, 64, 256, 256, B, None) == EUNSUP
    assert lib.dit_pack_weights(1, 0, A, 64, 256, 264, B + 1, None) == EALIGN
    assert lib.dit_gemm_q8_epilogue(A, B, C, 4, 512, 256, 2, D, 512, None) == EUNSUP
    assert lib.dit_gemm_q8_epilogue(A, B + 2, C, 4, 512, 256, 0, D, 512, None) == EALIGN
    assert lib.dit_gemm_q8_epilogue(A, None, C, 4, 512, 256, 0, D, 512, None) == EINVAL
    if not _has_gpu():
        assert lib.dit_quantize_act(1, A, 4, 256, 256, B, C, None) == EDEVICE
        assert lib.dit_quantize_act(1, A, 4, 384, 384, B, C, None) == EDEVICE
        assert lib.dit_quantize_act(3, A, 4, 256, 256, B, C + 1, None) == EDEVICE    # MXFP8 scales: any alignment
        assert lib.dit_pack_weights(2, 1, A, 128, 256, 256, B, None) == EDEVICE
        assert lib.dit_pack_weights(2, 2, A, 384, 256, 256, B, None) == EDEVICE      # FP8 for QK-RMSNorm
        assert lib.dit_pack_weights(3, 1, A, 128, 256, 256, B, None) == EDEVICE
        assert lib.dit_pack_weights(4, 1, A, 128, 256, 256, B, None) == EDEVICE
        assert lib.dit_quantize_act(4, A, 4, 256, 256, B, C, None) == EDEVICE
        assert lib.dit_gemm_q8_epilogue(A, B, C, 4, 512, 256, 1, D, 256, None) == EDEVICE


def _has_gpu():
    import torch
    return torch.cuda.device_count() > 0


def _any(fmt=3, a=A, s=B, w=C, M=64, N=512, K=256, epi=1, rms=None, out=D, ldo=256):
    return ditq._lib.dit_gemm_epilogue(fmt, a, s, w, M, N, K, epi, ctypes.byref(rms) if rms else None, out, ldo,
                                       None)


def test_gemm_any_format_validation():
    assert _any(fmt=0) == EINVAL
    assert _any(fmt=5) == EINVAL
    assert _any(out=None) == EINVAL
    assert _any(a=None) == EINVAL
    assert _any(epi=2) == EINVAL                                     # RMSNorm without params
    assert _any(fmt=2, epi=2) == EINVAL
    r = ditq.RmsNormParams(128, 1, A, B, 1e-6)
    assert _any(epi=0, rms=r, ldo=512) == EINVAL                     # params without RMSNorm
    assert _any(fmt=2, epi=2, rms=ditq.RmsNormParams(64, 2, A, B, 1e-6), N=384, ldo=384) == EUNSUP
    assert _any(K=320) == EUNSUP                                     # K % 128
    assert _any(fmt=2, N=576) == EUNSUP                              # gated needs N % 128
    assert _any(s=B + 4) == EALIGN                                   # MXFP8 scales: 16 B
    assert _any(fmt=2, s=B + 4) != EALIGN                            # FP8 row scales: 4 B is enough
    assert _any(fmt=2, s=B + 2) == EALIGN
    assert _any(ldo=255) == EALIGN
    if not _has_gpu():
        for fmt in (1, 2, 3, 4):
            assert _any(fmt=fmt) == EDEVICE
            assert _any(fmt=fmt, epi=0, ldo=512) == EDEVICE
            assert _any(fmt=fmt, epi=2, rms=r, N=384, ldo=384) == EDEVICE
            assert _any(fmt=fmt, epi=2, rms=ditq.RmsNormParams(256, 1, A, B, 1e-6), N=768, ldo=768) == EDEVICE


def _gr(fmt=1, a=A, s=B, w=C, M=64, N=512, K=256, gr="default", out=D, ldo=512):
    if gr == "default":
        gr = ditq.GateResidualParams(E, 512, F, 32)
    return ditq._lib.dit_gemm_gate_residual(fmt, a, s, w, M, N, K, ctypes.byref(gr) if gr else None, out, ldo,
                                            None)


def test_gate_residual_validation():
    P = ditq.GateResidualParams
    assert _gr(gr=None) == EINVAL
    assert _gr(out=None) == EINVAL
    assert _gr(gr=P(None, 512, F, 32)) == EINVAL
    assert _gr(gr=P(E, 512, None, 32)) == EINVAL
    assert _gr(gr=P(E, 512, F, 0)) == EINVAL
    assert _gr(gr=P(D + 1024, 512, F, 32)) == EINVAL                 # partial overlap with the output
    assert _gr(fmt=5) == EINVAL
    assert _gr(K=64) == EUNSUP                                       # K % 128
    assert _gr(gr=P(E + 8, 512, F, 32)) == EALIGN
    assert _gr(gr=P(E, 500, F, 32)) == EALIGN                         # ldr < N
    assert _gr(gr=P(E, 516, F, 32)) == EALIGN                         # ldr % 8
    assert _gr(gr=P(E, 512, F + 4, 32)) == EALIGN
    # the other entry points have no gated-residual parameters
    assert _q4(epi=4, ldo=512) == EINVAL
    assert ditq._lib.dit_gemm_q8_epilogue(A, B, C, 4, 512, 256, 4, D, 512, None) == EUNSUP
    assert _any(epi=4, ldo=512) == EINVAL
    assert ditq.dit_packed_weight_bytes(1, 4, 512, 256) == ditq.dit_packed_weight_bytes(1, 0, 512, 256)
    assert ditq.dit_packed_weight_bytes(3, 3, 512, 256) == ditq.dit_packed_weight_bytes(3, 0, 512, 256)
    if not _has_gpu():
        for fmt in (1, 2, 3, 4):
            assert _gr(fmt=fmt) == EDEVICE
            assert _gr(fmt=fmt, gr=P(D, 512, F, 7), out=D) == EDEVICE     # in place
            assert _any(fmt=fmt, epi=3, ldo=512) == EDEVICE               # GELU-tanh
        assert _q4(epi=3, ldo=512) == EDEVICE
        assert ditq._lib.dit_gemm_q8_epilogue(A, B, C, 4, 512, 256, 3, D, 512, None) == EDEVICE


def test_measurement_entry_points_validation():
    gs = ditq._lib.dit_gated_silu_bf16
    assert gs(None, 64, 512, 512, D, 256, None) == EINVAL
    assert gs(A, 64, 512, 512, None, 256, None) == EINVAL
    assert gs(A, 0, 512, 512, D, 256, None) == EINVAL
    assert gs(A, 64, -16, 512, D, 256, None) == EINVAL
    assert gs(A, 64, 520, 520, D, 260, None) == EUNSUP               # N % 16
    assert gs(A + 8, 64, 512, 512, D, 256, None) == EALIGN
    assert gs(A, 64, 512, 512, D + 4, 256, None) == EALIGN
    assert gs(A, 64, 512, 500, D, 256, None) == EALIGN               # ldc < N
    assert gs(A, 64, 512, 512, D, 248, None) == EALIGN               # ldo < N/2
    assert gs(A, 64, 512, 516, D, 256, None) == EALIGN               # ldc % 8
    pr = ditq._lib.dit_mfma_fp4_probe
    assert pr(256, 100, None, None) == EINVAL
    assert pr(0, 100, A, None) == EINVAL
    assert pr(65536, 100, A, None) == EINVAL
    assert pr(256, 0, A, None) == EINVAL
    assert pr(256, (1 << 20) + 1, A, None) == EINVAL
    assert pr(256, 100, A + 4, None) == EALIGN
    if not _has_gpu():
        assert gs(A, 64, 512, 512, D, 256, None) == EDEVICE
        assert pr(256, 100, A, None) == EDEVICE


def _blob_bytes(fmt, epi, N, K):
    """A blob of the documented size with a header as the packer writes it (the
    payload is zero: these tests only exercise the header checks)."""
    nbytes = ditq.dit_packed_weight_bytes(fmt, epi, N, K)
    Np = (N + 255) // 256 * 256
    b = np.zeros(nbytes, dtype=np.uint8)
    b[:28].view("<u4")[:] = [0x51544944, 2, fmt, epi, N, K, Np]
    b[32:56].view("<u8")[:] = [256, 256 + Np * K // 2, nbytes]
    return b


def test_packed_blob_save_load_header_checks(tmp_path):
    b = _blob_bytes(1, 1, 512, 256)
    hdr = ditq.check_blob(b, 1, 1, 512, 256, nbytes=b.size)
    assert (hdr["fmt"], hdr["epi"], hdr["N"], hdr["K"], hdr["Np"]) == (1, 1, 512, 256, 512)
    path = tmp_path / "w.ditq"
    b.tofile(path)
    t = ditq.load_packed(path, fmt=1, epi=1, N=512, K=256, device="cpu")
    assert t.numel() == b.size and (t.numpy() == b).all()
    # a blob packed for identity serves every epilogue but gated-SiLU (same row order)
    c = _blob_bytes(1, 0, 512, 256)
    ditq.check_blob(c, 1, 3, 512, 256)
    bad = {"magic": (0, 0xDEADBEEF), "version": (1, 1)}
    for name, (i, v) in bad.items():
        x = b.copy()
        x[:28].view("<u4")[i] = v
        with pytest.raises(ValueError, match=name):
            ditq.check_blob(x)
    for kw, msg in [(dict(fmt=2), "format"), (dict(epi=0), "row order"), (dict(N=256), "N ="), (dict(K=512), "K =")]:
        with pytest.raises(ValueError, match=msg):
            ditq.check_blob(b, **kw)
    with pytest.raises(ValueError, match="row order"):
        ditq.check_blob(c, epi=1)
    b[:-1].tofile(tmp_path / "short.ditq")
    with pytest.raises(ValueError, match="truncated"):
        ditq.load_packed(tmp_path / "short.ditq", device="cpu")
    x = b.copy()
    x[48:56].view("<u8")[0] = 1234
    with pytest.raises(ValueError, match="inconsistent"):
        ditq.check_blob(x)
    # fields no packer writes: an unknown format, an impossible shape, an empty blob
    for i, v in [(2, 99), (4, 0xFFFFFFFF), (5, 0x80000000), (4, 0)]:
        x = b.copy()
        x[:28].view("<u4")[i] = v
        x[48:56].view("<u8")[0] = 0
        with pytest.raises(ValueError, match="inconsistent"):
            ditq.check_blob(x)


def _f32(fmt=1, a=A, s=B, w=C, M=64, N=512, K=256, epi=1, rms=None, gr=None, out=D, ldo=256):
    return ditq._lib.dit_gemm_epilogue_f32(fmt, a, s, w, M, N, K, epi, ctypes.byref(rms) if rms else None,
                                           ctypes.byref(gr) if gr else None, out, ldo, None)


def test_gemm_f32_debug_validation():
    P = ditq.GateResidualParams
    assert _f32(out=None) == EINVAL
    assert _f32(epi=2) == EINVAL                                     # RMSNorm without params
    assert _f32(epi=4, ldo=512) == EINVAL                            # gated residual without params
    assert _f32(epi=1, gr=P(E, 512, F, 32)) == EINVAL                # params without the gated residual
    assert _f32(epi=4, gr=P(D, 512, F, 32), ldo=512) == EINVAL       # the residual overlaps the fp32 output
    assert _f32(K=192) == EUNSUP
    assert _f32(out=D + 8) == EALIGN
    assert _f32(ldo=255) == EALIGN                                   # < output width
    assert _f32(ldo=258) == EALIGN                                   # fp32 rows: a multiple of 4 elements
    if not _has_gpu():
        assert _f32(ldo=260) == EDEVICE
        assert _f32(fmt=2, epi=0, ldo=512) == EDEVICE
        assert _f32(epi=4, gr=P(0x1000000, 512, 0x2000000, 32), ldo=512) == EDEVICE


def test_quantize_noalloc_validation():
    lib = ditq._lib
    assert lib.dit_quantize_act_noalloc(4, None, 4, 256, 256, B, C, None) == EINVAL
    assert lib.dit_quantize_act_noalloc(4, A, 4, 256, 256, B, None, None) == EINVAL
    assert lib.dit_quantize_act_noalloc(4, A, 0, 256, 256, B, C, None) == EINVAL
    assert lib.dit_quantize_act_noalloc(9, A, 4, 256, 256, B, C, None) == EINVAL
    assert lib.dit_quantize_act_noalloc(4, A, 4, 320, 320, B, C, None) == EUNSUP     # K % 128
    assert lib.dit_quantize_act_noalloc(4, A, 1 << 30, 4096, 4096, B, C, None) == EUNSUP   # beyond the code limit
    assert lib.dit_quantize_act_noalloc(4, A, 4, 256, 256, B, C + 4, None) == EALIGN
    assert lib.dit_quantize_act_noalloc(4, A + 2, 4, 256, 256, B, C, None) == EALIGN
    if not _has_gpu():
        for fmt in (1, 2, 3, 4):
            assert lib.dit_quantize_act_noalloc(fmt, A, 4, 256, 256, B, C, None) == EDEVICE
