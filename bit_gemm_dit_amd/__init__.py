"""Python binding of libditq (the fused low-bit DiT linear layer on MI355X).

Argument marshalling only: every step runs in the HIP kernels of libditq.so.
The functions named ``dit_*`` mirror the C ABI in include/ditq.h and
include/ditq_measure.h one to one and take raw device pointers (ints); the helpers below them take torch tensors and
use torch only for device memory and the current stream.

The library must have been built (``python bit_gemm_dit_amd/build.py``); import
fails loudly otherwise.  There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "FMT_FP4", "FMT_FP8", "FMT_MX8", "FMT_NV4", "EPI_IDENTITY", "EPI_GATED_SILU", "EPI_QK_RMSNORM", "EPI_GELU_TANH",
    "EPI_GATE_RESIDUAL", "DitError", "RmsNormParams", "GateResidualParams",
    "dit_packed_weight_bytes", "dit_act_code_bytes", "dit_act_scale_bytes", "dit_pack_weights",
    "dit_quantize_act", "dit_quantize_act_noalloc", "dit_gemm_q4_epilogue", "dit_gemm_q4_epilogue_q4", "dit_gemm_q8_epilogue",
    "dit_gemm_epilogue", "dit_gemm_gate_residual", "gemm_gate_residual", "dit_gemm_epilogue_f32",
    "dit_gated_silu_bf16", "dit_mfma_fp4_probe", "gated_silu", "mfma_fp4_probe",
    "dit_status_str", "dit_last_error", "pack_weights", "quantize_act", "gemm", "gemm_q4out", "linear",
    "library_path", "EXPORTED", "BLOB_MAGIC", "BLOB_VERSION", "blob_header", "check_blob", "save_packed",
    "load_packed",
]

FMT_FP4 = 1
FMT_FP8 = 2
FMT_MX8 = 3
FMT_NV4 = 4
EPI_IDENTITY = 0
EPI_GATED_SILU = 1
EPI_QK_RMSNORM = 2
EPI_GELU_TANH = 3
EPI_GATE_RESIDUAL = 4

_HERE = os.path.dirname(os.path.abspath(__file__))
# DITQ_LIB selects another build of the library, e.g. the CPU-only sanitizer build
# of the ABI layer (build.py --sanitize); the default is the in-tree libditq.so.
library_path = os.environ.get("DITQ_LIB") or os.path.join(_HERE, "libditq.so")

if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is missing: build it with `python bit_gemm_dit_amd/build.py` "
        "(there is no CPU fallback)")

# torch ships its own HIP runtime (soname libamdhip64.so.7, loaded by file name).
# Loading torch first makes the dynamic linker bind libditq.so to that same copy;
# loading libditq.so first would map a second runtime from /opt/rocm, and two
# runtimes in one process do not share the device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(library_path)


class RmsNormParams(ctypes.Structure):
    """dit_rmsnorm_params: head_dim, n_heads, gamma_q / gamma_k (device pointers), eps."""
    _fields_ = [("head_dim", ctypes.c_int), ("n_heads", ctypes.c_int), ("gamma_q", ctypes.c_void_p),
                ("gamma_k", ctypes.c_void_p), ("eps", ctypes.c_float)]


class GateResidualParams(ctypes.Structure):
    """dit_gate_residual_params: residual (device bf16), ldr, gate (device fp32), rows_per_gate."""
    _fields_ = [("residual", ctypes.c_void_p), ("ldr", ctypes.c_int), ("gate", ctypes.c_void_p),
                ("rows_per_gate", ctypes.c_int)]


_i, _p, _sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
_SIGS = {
    "dit_packed_weight_bytes": (_sz, [_i, _i, _i, _i]),
    "dit_act_code_bytes": (_sz, [_i, _i, _i]),
    "dit_act_scale_bytes": (_sz, [_i, _i, _i]),
    "dit_pack_weights": (_i, [_i, _i, _p, _i, _i, _i, _p, _p]),
    "dit_quantize_act": (_i, [_i, _p, _i, _i, _i, _p, _p, _p]),
    "dit_quantize_act_noalloc": (_i, [_i, _p, _i, _i, _i, _p, _p, _p]),
    "dit_gemm_q4_epilogue": (_i, [_p, _p, _p, _i, _i, _i, _i, ctypes.POINTER(RmsNormParams), _p, _i, _p]),
    "dit_gemm_q4_epilogue_q4": (_i, [_p, _p, _p, _i, _i, _i, _i, ctypes.POINTER(RmsNormParams), _p, _i, _p, _p,
                                     _p]),
    "dit_gemm_q8_epilogue": (_i, [_p, _p, _p, _i, _i, _i, _i, _p, _i, _p]),
    "dit_gemm_epilogue": (_i, [_i, _p, _p, _p, _i, _i, _i, _i, ctypes.POINTER(RmsNormParams), _p, _i, _p]),
    "dit_gemm_gate_residual": (_i, [_i, _p, _p, _p, _i, _i, _i, ctypes.POINTER(GateResidualParams), _p, _i, _p]),
    "dit_gemm_epilogue_f32": (_i, [_i, _p, _p, _p, _i, _i, _i, _i, ctypes.POINTER(RmsNormParams),
                                   ctypes.POINTER(GateResidualParams), _p, _i, _p]),
    "dit_gated_silu_bf16": (_i, [_p, _i, _i, _i, _p, _i, _p]),
    "dit_mfma_fp4_probe": (_i, [_i, _i, _p, _p]),
    "dit_status_str": (ctypes.c_char_p, [_i]),
    "dit_last_error": (ctypes.c_char_p, []),
}
EXPORTED = tuple(_SIGS)
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class DitError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = dit_last_error() if status == 4 else ""
        super().__init__(f"{where}: {dit_status_str(status)} (status {status})" + (f" [{detail}]" if detail else ""))


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DitError(status, where)


# ---------------------------------------------------------------- C ABI mirrors
def dit_status_str(status: int) -> str:
    return _lib.dit_status_str(status).decode()


def dit_last_error() -> str:
    return _lib.dit_last_error().decode()


def dit_packed_weight_bytes(fmt: int, epi: int, N: int, K: int) -> int:
    return _lib.dit_packed_weight_bytes(fmt, epi, N, K)


def dit_act_code_bytes(fmt: int, M: int, K: int) -> int:
    return _lib.dit_act_code_bytes(fmt, M, K)


def dit_act_scale_bytes(fmt: int, M: int, K: int) -> int:
    return _lib.dit_act_scale_bytes(fmt, M, K)


def dit_pack_weights(fmt, epi, w_ptr, N, K, ldw, packed_ptr, stream=None) -> None:
    _check(_lib.dit_pack_weights(fmt, epi, w_ptr, N, K, ldw, packed_ptr, stream), "dit_pack_weights")


def dit_quantize_act(fmt, x_ptr, M, K, ldx, codes_ptr, scales_ptr, stream=None) -> None:
    _check(_lib.dit_quantize_act(fmt, x_ptr, M, K, ldx, codes_ptr, scales_ptr, stream), "dit_quantize_act")


def dit_quantize_act_noalloc(fmt, x_ptr, M, K, ldx, codes_ptr, scales_ptr, stream=None) -> None:
    _check(_lib.dit_quantize_act_noalloc(fmt, x_ptr, M, K, ldx, codes_ptr, scales_ptr, stream),
           "dit_quantize_act_noalloc")


def dit_gemm_q4_epilogue(a_codes, a_scales, w_packed, M, N, K, epi, rms, out, ldo, stream=None) -> None:
    rp = ctypes.byref(rms) if rms is not None else None
    _check(_lib.dit_gemm_q4_epilogue(a_codes, a_scales, w_packed, M, N, K, epi, rp, out, ldo, stream),
           "dit_gemm_q4_epilogue")


def dit_gemm_q4_epilogue_q4(a_codes, a_scales, w_packed, M, N, K, epi, rms, out, ldo, out_codes, out_scales,
                            stream=None) -> None:
    rp = ctypes.byref(rms) if rms is not None else None
    _check(_lib.dit_gemm_q4_epilogue_q4(a_codes, a_scales, w_packed, M, N, K, epi, rp, out, ldo, out_codes,
                                        out_scales, stream), "dit_gemm_q4_epilogue_q4")


def dit_gemm_q8_epilogue(a_codes, a_scales, w_packed, M, N, K, epi, out, ldo, stream=None) -> None:
    _check(_lib.dit_gemm_q8_epilogue(a_codes, a_scales, w_packed, M, N, K, epi, out, ldo, stream),
           "dit_gemm_q8_epilogue")


def dit_gemm_epilogue(fmt, a_codes, a_scales, w_packed, M, N, K, epi, rms, out, ldo, stream=None) -> None:
    rp = ctypes.byref(rms) if rms is not None else None
    _check(_lib.dit_gemm_epilogue(fmt, a_codes, a_scales, w_packed, M, N, K, epi, rp, out, ldo, stream),
           "dit_gemm_epilogue")


def dit_gemm_gate_residual(fmt, a_codes, a_scales, w_packed, M, N, K, gr, out, ldo, stream=None) -> None:
    gp = ctypes.byref(gr) if gr is not None else None
    _check(_lib.dit_gemm_gate_residual(fmt, a_codes, a_scales, w_packed, M, N, K, gp, out, ldo, stream),
           "dit_gemm_gate_residual")


def dit_gemm_epilogue_f32(fmt, a_codes, a_scales, w_packed, M, N, K, epi, rms, gr, out_f32, ldo,
                          stream=None) -> None:
    rp = ctypes.byref(rms) if rms is not None else None
    gp = ctypes.byref(gr) if gr is not None else None
    _check(_lib.dit_gemm_epilogue_f32(fmt, a_codes, a_scales, w_packed, M, N, K, epi, rp, gp, out_f32, ldo, stream),
           "dit_gemm_epilogue_f32")


def dit_gated_silu_bf16(c, M, N, ldc, out, ldo, stream=None) -> None:
    _check(_lib.dit_gated_silu_bf16(c, M, N, ldc, out, ldo, stream), "dit_gated_silu_bf16")


def dit_mfma_fp4_probe(workgroups, iters, out_u64, stream=None) -> None:
    _check(_lib.dit_mfma_fp4_probe(workgroups, iters, out_u64, stream), "dit_mfma_fp4_probe")


# ---------------------------------------------------------------- torch helpers
def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ld(t) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit stride along the last dimension")
    return t.stride(0)


def pack_weights(w, fmt: int, epi: int):
    """bf16 weights [N, K] (torch Linear layout) -> packed blob (uint8 device tensor)."""
    import torch
    N, K = w.shape
    nbytes = dit_packed_weight_bytes(fmt, epi, N, K)
    if nbytes == 0:
        raise DitError(2, "dit_packed_weight_bytes")
    blob = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    dit_pack_weights(fmt, epi, w.data_ptr(), N, K, _ld(w), blob.data_ptr(), _stream())
    return blob


BLOB_MAGIC = 0x51544944          # "DITQ", the first u32 of a packed blob
BLOB_VERSION = 2
_HEADER_FIELDS = ("magic", "version", "fmt", "epi", "N", "K", "Np")


def blob_header(data) -> dict:
    """The header fields of a packed blob (the layout in include/ditq.h): magic,
    version, fmt, epi, N, K, Np and the total byte count.  `data` is the blob as a
    torch uint8 tensor (device or host) or as bytes / a NumPy uint8 array; only its
    first 64 bytes are read (copied to the host)."""
    import numpy as np
    if hasattr(data, "cpu"):
        data = data[:64].cpu().numpy()
    h = np.frombuffer(bytes(memoryview(np.ascontiguousarray(data[:64], dtype=np.uint8))), dtype=np.uint8)
    if h.size < 64:
        raise ValueError("packed blob shorter than its header")
    u32 = h[:28].view("<u4")
    out = {k: int(v) for k, v in zip(_HEADER_FIELDS, u32)}
    out["bytes"] = int(h[48:56].view("<u8")[0])
    return out


def check_blob(data, fmt=None, epi=None, N=None, K=None, nbytes=None) -> dict:
    """Validate a packed blob's header against the call it is meant for; returns the
    header.  Raises ValueError on a foreign or truncated blob, another layout version,
    or a format / shape / row order that does not match.  Blobs packed for
    gated-SiLU have their own row order; all other epilogues share one."""
    hdr = blob_header(data)
    if hdr["magic"] != BLOB_MAGIC:
        raise ValueError(f"not a packed weight blob (magic {hdr['magic']:#x})")
    if hdr["version"] != BLOB_VERSION:
        raise ValueError(f"blob layout version {hdr['version']}, this library writes {BLOB_VERSION}")
    fields_ok = all(0 < hdr[k] < 2 ** 31 for k in ("fmt", "N", "K")) and 0 <= hdr["epi"] < 2 ** 31
    expected = dit_packed_weight_bytes(hdr["fmt"], hdr["epi"], hdr["N"], hdr["K"]) if fields_ok else 0
    if expected == 0 or expected != hdr["bytes"]:
        raise ValueError("blob header is inconsistent (format, shape or byte count)")
    if nbytes is not None and nbytes < hdr["bytes"]:
        raise ValueError(f"blob truncated: {nbytes} of {hdr['bytes']} bytes")
    if fmt is not None and hdr["fmt"] != fmt:
        raise ValueError(f"blob packed for format {hdr['fmt']}, not {fmt}")
    if epi is not None and (hdr["epi"] == EPI_GATED_SILU) != (epi == EPI_GATED_SILU):
        raise ValueError(f"blob packed for epilogue {hdr['epi']}: row order differs from epilogue {epi}")
    if N is not None and hdr["N"] != N:
        raise ValueError(f"blob packed for N = {hdr['N']}, not {N}")
    if K is not None and hdr["K"] != K:
        raise ValueError(f"blob packed for K = {hdr['K']}, not {K}")
    return hdr


def save_packed(blob, path) -> dict:
    """Write a packed blob (device tensor) to a file, after checking its header."""
    import numpy as np
    host = blob.cpu().numpy()
    hdr = check_blob(host, nbytes=host.size)
    np.ascontiguousarray(host[:hdr["bytes"]], dtype=np.uint8).tofile(path)
    return hdr


def load_packed(path, fmt=None, epi=None, N=None, K=None, device="cuda"):
    """Read a blob written by save_packed and check its header against the expected
    format, epilogue row order and shape before it is uploaded; returns a uint8
    tensor on `device`."""
    import numpy as np
    import torch
    data = np.fromfile(path, dtype=np.uint8)
    check_blob(data, fmt, epi, N, K, nbytes=data.size)
    return torch.from_numpy(data).to(device)


def quantize_act(x, fmt: int):
    """bf16 activations [M, K] -> (codes, scales) device tensors."""
    import torch
    M, K = x.shape
    cb, sb = dit_act_code_bytes(fmt, M, K), dit_act_scale_bytes(fmt, M, K)
    if cb == 0:
        raise DitError(2, "dit_act_code_bytes")
    # K-panel-major layouts (include/ditq.h): shapes are [panels, M, bytes per panel row]
    if fmt == FMT_FP4:
        codes = torch.empty((K // 128, M, 64), dtype=torch.uint8, device=x.device)
        scales = torch.empty((K // 128, M, 4), dtype=torch.uint8, device=x.device)
    elif fmt == FMT_MX8:
        codes = torch.empty((K // 64, M, 64), dtype=torch.uint8, device=x.device)
        scales = torch.empty((K // 128, M, 4), dtype=torch.uint8, device=x.device)
    elif fmt == FMT_NV4:
        # block scales [K/128][M][8], then a 16-byte tail holding the tensor scale
        codes = torch.empty((K // 128, M, 64), dtype=torch.uint8, device=x.device)
        scales = torch.empty((sb,), dtype=torch.uint8, device=x.device)
    else:
        codes = torch.empty((K // 64, M, 64), dtype=torch.uint8, device=x.device)
        scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    assert codes.numel() * codes.element_size() == cb and scales.numel() * scales.element_size() == sb
    dit_quantize_act(fmt, x.data_ptr(), M, K, _ld(x), codes.data_ptr(), scales.data_ptr(), _stream())
    return codes, scales


def gemm(codes, scales, blob, N: int, K: int, fmt: int, epi: int, rms: RmsNormParams | None = None, out=None):
    """Fused GEMM + epilogue on quantized activations; returns the bf16 output [M, N or N/2]."""
    import torch
    M = codes.shape[1]
    width = N // 2 if epi == EPI_GATED_SILU else N
    if out is None:
        out = torch.empty((M, width), dtype=torch.bfloat16, device=codes.device)
    if fmt == FMT_FP4:
        dit_gemm_q4_epilogue(codes.data_ptr(), scales.data_ptr(), blob.data_ptr(), M, N, K, epi, rms,
                             out.data_ptr(), _ld(out), _stream())
    elif fmt == FMT_FP8 and epi != EPI_QK_RMSNORM:
        dit_gemm_q8_epilogue(codes.data_ptr(), scales.data_ptr(), blob.data_ptr(), M, N, K, epi,
                             out.data_ptr(), _ld(out), _stream())
    else:
        dit_gemm_epilogue(fmt, codes.data_ptr(), scales.data_ptr(), blob.data_ptr(), M, N, K, epi, rms,
                          out.data_ptr(), _ld(out), _stream())
    return out


def gemm_q4out(codes, scales, blob, N: int, K: int, epi: int, rms: RmsNormParams | None = None,
               with_bf16: bool = False):
    """FP4 GEMM + epilogue whose output is quantized to FP4 for the next GEMM.

    Returns (out_codes, out_scales) in the activation layout of quantize_act (ready
    to be the next layer's input), plus the bf16 output when with_bf16.
    """
    import torch
    M = codes.shape[1]
    width = N // 2 if epi == EPI_GATED_SILU else N
    q_codes = torch.empty((width // 128, M, 64), dtype=torch.uint8, device=codes.device)
    q_scales = torch.empty((width // 128, M, 4), dtype=torch.uint8, device=codes.device)
    out = torch.empty((M, width), dtype=torch.bfloat16, device=codes.device) if with_bf16 else None
    dit_gemm_q4_epilogue_q4(codes.data_ptr(), scales.data_ptr(), blob.data_ptr(), M, N, K, epi, rms,
                            out.data_ptr() if out is not None else None, _ld(out) if out is not None else 0,
                            q_codes.data_ptr(), q_scales.data_ptr(), _stream())
    return (q_codes, q_scales, out) if with_bf16 else (q_codes, q_scales)


def gemm_gate_residual(codes, scales, blob, N: int, K: int, fmt: int, residual, gate, rows_per_gate: int,
                       out=None):
    """out = residual + gate[row // rows_per_gate] * (A W^T), bf16 [M, N]; `out` may be
    `residual` itself (an in-place update of the residual stream)."""
    import torch
    M = codes.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=codes.device)
    gr = GateResidualParams(residual.data_ptr(), _ld(residual), gate.data_ptr(), rows_per_gate)
    dit_gemm_gate_residual(fmt, codes.data_ptr(), scales.data_ptr(), blob.data_ptr(), M, N, K, gr,
                           out.data_ptr(), _ld(out), _stream())
    return out


def linear(x, blob, N: int, fmt: int, epi: int, rms: RmsNormParams | None = None, out=None):
    """The whole layer: quantize x on the fly, then the fused GEMM + epilogue."""
    codes, scales = quantize_act(x, fmt)
    return gemm(codes, scales, blob, N, x.shape[1], fmt, epi, rms=rms, out=out)


def gated_silu(c, out=None):
    """Gated-SiLU as a separate pass over a bf16 GEMM output c = [gate | up] [M, N];
    returns bf16 [M, N/2] (the unfused form of EPI_GATED_SILU)."""
    import torch
    M, N = c.shape
    if out is None:
        out = torch.empty((M, N // 2), dtype=torch.bfloat16, device=c.device)
    dit_gated_silu_bf16(c.data_ptr(), M, N, _ld(c), out.data_ptr(), _ld(out), _stream())
    return out


def mfma_fp4_probe(workgroups: int, iters: int):
    """Enqueue the matrix-core probe; returns the uint64 device tensor [workgroups, 2]
    of (loop cycles of wave 0, checksum) per workgroup."""
    import torch
    out = torch.zeros((workgroups, 2), dtype=torch.int64, device="cuda")
    dit_mfma_fp4_probe(workgroups, iters, out.data_ptr(), _stream())
    return out


def rmsnorm_params(gamma_q, gamma_k, n_heads: int, eps: float) -> RmsNormParams:
    """Build the RMSNorm parameter struct from fp32 device tensors (kept alive by the caller)."""
    return RmsNormParams(gamma_q.numel(), n_heads, gamma_q.data_ptr(), gamma_k.data_ptr(), eps)
