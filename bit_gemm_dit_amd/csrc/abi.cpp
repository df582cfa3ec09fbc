// C ABI of the fused low-bit linear layer: argument validation and dispatch.
//
// Every check runs on the host before any HIP call (so the error paths can be
// exercised without a device); the kernels themselves live in quant.hip,
// pack.hip, gemm.hip and measure.hip.  The entry points and their contracts are
// declared and documented in include/ditq.h and include/ditq_measure.h.
#include "ditq.h"
#include "ditq_measure.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdio>
#include <cstring>

#include "common.hpp"

namespace {

using ditq::FMT_FP4;
using ditq::FMT_FP8;
using ditq::FMT_MX8;
using ditq::FMT_NV4;

// The value of an enum argument as an int.  A C caller (or ctypes) may pass any int
// for an enum parameter, and in C++ reading an enum object whose value lies outside
// the enumeration's range is undefined behaviour; so the entry points copy the
// argument's bytes instead and work with ints.
template <class E>
int raw(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool valid_fmt(int f) {
  return f == DIT_FMT_FP4_E2M1_MX32 || f == DIT_FMT_FP8_E4M3_ROWCOL || f == DIT_FMT_FP8_E4M3_MX32 ||
         f == DIT_FMT_FP4_E2M1_NV16;
}
bool valid_epi(int e) {
  return e == DIT_EPI_IDENTITY || e == DIT_EPI_GATED_SILU || e == DIT_EPI_QK_RMSNORM || e == DIT_EPI_GELU_TANH ||
         e == DIT_EPI_GATE_RESIDUAL;
}

// Shapes the kernels implement.  K: whole 128-element k-steps (one 128-byte FP4
// scale record per 32 weight rows, one 64-byte activation panel row per token);
// N: whole 64-row weight groups (128 for gated-SiLU so each 64-row packed group
// holds 32 gate/up pairs).  Byte counts stay below 2^31 so that 32-bit buffer
// offsets cover every tensor plus one tile of ragged rows, and the k-steps the
// GEMM pads K with (at most three, reading zeros past the end).
bool shape_ok(int fmt, int epi, int N, int K) {
  if (K % 128 != 0 || N % 64 != 0) return false;
  if (epi == DIT_EPI_GATED_SILU && N % 128 != 0) return false;
  const size_t Np = (size_t)ditq::padded_rows(N);
  const size_t code_bytes = ditq::is_fp4_codes(fmt) ? Np * K / 2 : Np * K;
  return code_bytes < (1ull << 31);
}
bool rows_ok(int fmt, int M, int K) {
  const size_t row = ditq::is_fp4_codes(fmt) ? (size_t)K / 2 : (size_t)K;
  return ((size_t)M + 256) * row < (1ull << 31);
}

// Detail of the most recent DIT_EDEVICE on this thread (see dit_last_error).
thread_local char g_last_error[256] = "";

dit_status device_error(const char* what, hipError_t e) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return DIT_EDEVICE;
}

// DIT_OK if the current device is a gfx950, DIT_EDEVICE otherwise.  Cached per device id.
dit_status check_device() {
  static std::atomic<int> ok_dev{-1};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return device_error("hipGetDevice", e);
  if (ok_dev.load(std::memory_order_relaxed) == dev) return DIT_OK;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return device_error("hipGetDeviceProperties", e);
  const char* arch = prop.gcnArchName;
  if (!(arch[0] == 'g' && arch[1] == 'f' && arch[2] == 'x' && arch[3] == '9' && arch[4] == '5' && arch[5] == '0')) {
    std::snprintf(g_last_error, sizeof g_last_error, "device %d is %s, not gfx950", dev, arch);
    return DIT_EDEVICE;
  }
  ok_dev.store(dev, std::memory_order_relaxed);
  // A failed query made by other code earlier on this thread stays pending in
  // hipGetLastError; drop it so that the check after our launch sees only ours.
  (void)hipGetLastError();
  return DIT_OK;
}

dit_status launched(hipError_t e) { return e == hipSuccess ? DIT_OK : device_error("kernel launch", e); }

}  // namespace

extern "C" {

size_t dit_packed_weight_bytes(dit_fmt fmt_, dit_epi epi_, int N, int K) {
  const int fmt = raw(fmt_), epi = raw(epi_);
  if (!valid_fmt(fmt) || !valid_epi(epi) || N <= 0 || K <= 0) return 0;
  if (!shape_ok(fmt, epi, N, K)) return 0;
  return ditq::blob_total_bytes(fmt, ditq::padded_rows(N), K);
}

size_t dit_act_code_bytes(dit_fmt fmt_, int M, int K) {
  const int fmt = raw(fmt_);
  if (!valid_fmt(fmt) || M <= 0 || K <= 0 || K % 128 != 0) return 0;
  return ditq::is_fp4_codes(fmt) ? (size_t)M * K / 2 : (size_t)M * K;
}

size_t dit_act_scale_bytes(dit_fmt fmt_, int M, int K) {
  const int fmt = raw(fmt_);
  if (!valid_fmt(fmt) || M <= 0 || K <= 0 || K % 128 != 0) return 0;
  if (fmt == DIT_FMT_FP8_E4M3_ROWCOL) return (size_t)M * 4;
  if (fmt == DIT_FMT_FP4_E2M1_NV16) return ditq::nv4_act_tail(M, K) + ditq::kNvTailBytes + ditq::kNvPartialBytes;
  return (size_t)M * K / 32;
}

dit_status dit_pack_weights(dit_fmt fmt_, dit_epi epi_, const void* w_bf16, int N, int K, int ldw, void* packed,
                            void* stream) {
  const int fmt = raw(fmt_), epi = raw(epi_);
  if (!valid_fmt(fmt) || !valid_epi(epi) || !w_bf16 || !packed || N <= 0 || K <= 0) return DIT_EINVAL;
  if (!shape_ok(fmt, epi, N, K)) return DIT_EUNSUPPORTED;
  if (!aligned16(w_bf16) || !aligned16(packed) || ldw < K || ldw % 8 != 0) return DIT_EALIGN;
  if (dit_status s = check_device()) return s;
  (void)hipGetLastError();
  return launched(ditq::launch_pack(fmt, epi, static_cast<const uint16_t*>(w_bf16), N, K, ldw,
                                    static_cast<uint8_t*>(packed), static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {
// Checks and launch of both quantizer entry points.  static_work: NVFP4 keeps its
// tensor-maximum work space in the library's static array instead of the scale
// buffer's tail.
dit_status quantize_any(int fmt, const void* x_bf16, int M, int K, int ldx, void* codes, void* scales,
                        bool static_work, void* stream) {
  if (!valid_fmt(fmt) || !x_bf16 || !codes || !scales || M <= 0 || K <= 0) return DIT_EINVAL;
  if (K % 128 != 0 || !rows_ok(fmt, M, K)) return DIT_EUNSUPPORTED;
  if (!aligned16(x_bf16) || !aligned16(codes) || ldx < K || ldx % 8 != 0) return DIT_EALIGN;
  if (fmt == DIT_FMT_FP8_E4M3_ROWCOL && !aligned(scales, 4)) return DIT_EALIGN;
  if (fmt == DIT_FMT_FP4_E2M1_NV16 && !aligned16(scales)) return DIT_EALIGN;
  if (dit_status s = check_device()) return s;
  (void)hipGetLastError();
  const auto x = static_cast<const uint16_t*>(x_bf16);
  const auto c = static_cast<uint8_t*>(codes);
  const auto st = static_cast<hipStream_t>(stream);
  if (fmt == DIT_FMT_FP4_E2M1_MX32)
    return launched(ditq::launch_quant_fp4(x, M, K, ldx, c, static_cast<uint8_t*>(scales), st));
  if (fmt == DIT_FMT_FP8_E4M3_MX32)
    return launched(ditq::launch_quant_mx8(x, M, K, ldx, c, static_cast<uint8_t*>(scales), st));
  if (fmt == DIT_FMT_FP4_E2M1_NV16) {
    if (static_work)
      return launched(ditq::launch_quant_nv4_static(x, M, K, ldx, c, static_cast<uint8_t*>(scales), st));
    return launched(ditq::launch_quant_nv4(x, M, K, ldx, c, static_cast<uint8_t*>(scales), nullptr, st));
  }
  return launched(ditq::launch_quant_fp8(x, M, K, ldx, c, static_cast<float*>(scales), st));
}
}  // namespace

extern "C" {

dit_status dit_quantize_act(dit_fmt fmt, const void* x_bf16, int M, int K, int ldx, void* codes, void* scales,
                            void* stream) {
  return quantize_any(raw(fmt), x_bf16, M, K, ldx, codes, scales, false, stream);
}

dit_status dit_quantize_act_noalloc(dit_fmt fmt, const void* x_bf16, int M, int K, int ldx, void* codes,
                                    void* scales, void* stream) {
  return quantize_any(raw(fmt), x_bf16, M, K, ldx, codes, scales, true, stream);
}

namespace {
// Checks and launch shared by every GEMM entry point.  out_codes set: the FP4
// quantization of the output is written too (FP4 only), and out_bf16 may be null.
dit_status gemm_any(int fmt, const void* a_codes, const void* a_scales, const void* w_packed, int M, int N, int K,
                    int epi, const dit_rmsnorm_params* rms, const dit_gate_residual_params* gr,
                    void* out_bf16, int ldo, void* out_codes, void* out_scales, float* out_f32, void* stream) {
  const bool quantized = out_codes != nullptr;
  if (!valid_fmt(fmt) || !a_codes || !a_scales || !w_packed || M <= 0 || N <= 0 || K <= 0 || !valid_epi(epi))
    return DIT_EINVAL;
  if (!quantized && !out_bf16 && !out_f32) return DIT_EINVAL;
  if (quantized && !out_scales) return DIT_EINVAL;
  if ((epi == DIT_EPI_QK_RMSNORM) != (rms != nullptr)) return DIT_EINVAL;
  if ((epi == DIT_EPI_GATE_RESIDUAL) != (gr != nullptr)) return DIT_EINVAL;
  if (gr) {
    if (!gr->residual || !gr->gate || gr->rows_per_gate <= 0 || !(out_bf16 || out_f32)) return DIT_EINVAL;
    // the residual may be the bf16 output itself (an in-place update), but no other overlap
    const size_t esz = out_f32 ? 4 : 2;
    const uintptr_t r0 = reinterpret_cast<uintptr_t>(gr->residual);
    const uintptr_t o0 = reinterpret_cast<uintptr_t>(out_f32 ? static_cast<void*>(out_f32) : out_bf16);
    const uintptr_t r1 = r0 + 2 * ((size_t)(M - 1) * (size_t)gr->ldr + N);
    const uintptr_t o1 = o0 + esz * ((size_t)(M - 1) * (size_t)ldo + N);
    const bool same = !out_f32 && r0 == o0 && gr->ldr == ldo;
    if (!same && r0 < o1 && o0 < r1) return DIT_EINVAL;
  }
  if (rms) {
    if (!rms->gamma_q || !rms->gamma_k || rms->n_heads <= 0 || !(rms->eps > 0.0f)) return DIT_EINVAL;
    if ((long long)N != 3LL * rms->n_heads * rms->head_dim) return DIT_EINVAL;
    if (rms->head_dim != 128 && rms->head_dim != 256) return DIT_EUNSUPPORTED;
  }
  if (!shape_ok(fmt, epi, N, K) || !rows_ok(fmt, M, K)) return DIT_EUNSUPPORTED;
  const int width = epi == DIT_EPI_GATED_SILU ? N / 2 : N;
  // the quantized output is an FP4 activation of M rows and K' = width columns
  if (quantized && (fmt != FMT_FP4 || width % 256 != 0 || !rows_ok(FMT_FP4, M, width))) return DIT_EUNSUPPORTED;
  if (!aligned16(a_codes) || !aligned16(w_packed)) return DIT_EALIGN;
  if (fmt == FMT_FP8 ? !aligned(a_scales, 4) : !aligned16(a_scales)) return DIT_EALIGN;
  if (out_bf16 && (!aligned16(out_bf16) || ldo < width || ldo % 8 != 0)) return DIT_EALIGN;
  if (out_f32 && (!aligned16(out_f32) || ldo < width || ldo % 4 != 0)) return DIT_EALIGN;
  if (quantized && (!aligned16(out_codes) || !aligned16(out_scales))) return DIT_EALIGN;
  if (rms && (!aligned16(rms->gamma_q) || !aligned16(rms->gamma_k))) return DIT_EALIGN;
  if (gr && (!aligned16(gr->residual) || !aligned16(gr->gate) || gr->ldr < N || gr->ldr % 8 != 0))
    return DIT_EALIGN;
  if (dit_status s = check_device()) return s;
  (void)hipGetLastError();
  ditq::RmsArgs r{};
  if (rms) r = ditq::RmsArgs{rms->head_dim, rms->n_heads, rms->gamma_q, rms->gamma_k, rms->eps};
  ditq::ResidualArgs g{};
  if (gr) g = ditq::ResidualArgs{static_cast<const uint16_t*>(gr->residual), gr->ldr, gr->gate, gr->rows_per_gate};
  return launched(ditq::launch_gemm(fmt, static_cast<const uint8_t*>(a_codes), a_scales,
                                    static_cast<const uint8_t*>(w_packed), M, N, K, epi, rms ? &r : nullptr,
                                    gr ? &g : nullptr, static_cast<uint16_t*>(out_bf16), ldo,
                                    static_cast<uint8_t*>(out_codes), static_cast<uint8_t*>(out_scales), out_f32,
                                    static_cast<hipStream_t>(stream)));
}
}  // namespace

dit_status dit_gemm_q4_epilogue(const void* a_codes, const void* a_scales, const void* w_packed, int M, int N,
                                int K, dit_epi epi_, const dit_rmsnorm_params* rms, void* out_bf16, int ldo,
                                void* stream) {
  const int epi = raw(epi_);
  if (!out_bf16) return DIT_EINVAL;
  return gemm_any(FMT_FP4, a_codes, a_scales, w_packed, M, N, K, epi, rms, nullptr, out_bf16, ldo, nullptr,
                  nullptr, nullptr, stream);
}

dit_status dit_gemm_q4_epilogue_q4(const void* a_codes, const void* a_scales, const void* w_packed, int M, int N,
                                   int K, dit_epi epi_, const dit_rmsnorm_params* rms, void* out_bf16, int ldo,
                                   void* out_codes, void* out_scales, void* stream) {
  const int epi = raw(epi_);
  if (!out_codes || !out_scales) return DIT_EINVAL;
  return gemm_any(FMT_FP4, a_codes, a_scales, w_packed, M, N, K, epi, rms, nullptr, out_bf16, ldo, out_codes,
                  out_scales, nullptr, stream);
}

dit_status dit_gemm_q8_epilogue(const void* a_codes, const float* a_scales, const void* w_packed, int M, int N,
                                int K, dit_epi epi_, void* out_bf16, int ldo, void* stream) {
  const int epi = raw(epi_);
  if (!a_codes || !a_scales || !w_packed || !out_bf16 || M <= 0 || N <= 0 || K <= 0 || !valid_epi(epi))
    return DIT_EINVAL;
  // no parameters for RMSNorm or the gated residual here
  if (epi == DIT_EPI_QK_RMSNORM || epi == DIT_EPI_GATE_RESIDUAL) return DIT_EUNSUPPORTED;
  return gemm_any(FMT_FP8, a_codes, a_scales, w_packed, M, N, K, epi, nullptr, nullptr, out_bf16, ldo, nullptr,
                  nullptr, nullptr, stream);
}

dit_status dit_gemm_epilogue(dit_fmt fmt_, const void* a_codes, const void* a_scales, const void* w_packed, int M,
                             int N, int K, dit_epi epi_, const dit_rmsnorm_params* rms, void* out_bf16, int ldo,
                             void* stream) {
  const int fmt = raw(fmt_), epi = raw(epi_);
  if (!out_bf16) return DIT_EINVAL;
  return gemm_any(fmt, a_codes, a_scales, w_packed, M, N, K, epi, rms, nullptr, out_bf16, ldo, nullptr, nullptr,
                  nullptr, stream);
}

dit_status dit_gemm_gate_residual(dit_fmt fmt_, const void* a_codes, const void* a_scales, const void* w_packed,
                                  int M, int N, int K, const dit_gate_residual_params* gr, void* out_bf16, int ldo,
                                  void* stream) {
  const int fmt = raw(fmt_);
  if (!gr || !out_bf16) return DIT_EINVAL;
  return gemm_any(fmt, a_codes, a_scales, w_packed, M, N, K, DIT_EPI_GATE_RESIDUAL, nullptr, gr, out_bf16, ldo,
                  nullptr, nullptr, nullptr, stream);
}

dit_status dit_gemm_epilogue_f32(dit_fmt fmt_, const void* a_codes, const void* a_scales, const void* w_packed,
                                 int M, int N, int K, dit_epi epi_, const dit_rmsnorm_params* rms,
                                 const dit_gate_residual_params* gr, float* out_f32, int ldo, void* stream) {
  const int fmt = raw(fmt_), epi = raw(epi_);
  if (!out_f32) return DIT_EINVAL;
  return gemm_any(fmt, a_codes, a_scales, w_packed, M, N, K, epi, rms, gr, nullptr, ldo, nullptr, nullptr, out_f32,
                  stream);
}

dit_status dit_gated_silu_bf16(const void* c_bf16, int M, int N, int ldc, void* out_bf16, int ldo,
                               void* stream) {
  if (!c_bf16 || !out_bf16 || M <= 0 || N <= 0) return DIT_EINVAL;
  if (N % 16 != 0 || (long long)M * (N / 16) >= (1LL << 31)) return DIT_EUNSUPPORTED;
  if (!aligned16(c_bf16) || !aligned16(out_bf16) || ldc < N || ldo < N / 2 || ldc % 8 != 0 || ldo % 8 != 0)
    return DIT_EALIGN;
  if (dit_status s = check_device()) return s;
  (void)hipGetLastError();
  return launched(ditq::launch_gated_silu(static_cast<const uint16_t*>(c_bf16), M, N, ldc,
                                          static_cast<uint16_t*>(out_bf16), ldo, static_cast<hipStream_t>(stream)));
}

dit_status dit_mfma_fp4_probe(int workgroups, int iters, void* out_u64, void* stream) {
  if (!out_u64 || workgroups < 1 || workgroups > 65535 || iters < 1 || iters > (1 << 20)) return DIT_EINVAL;
  if (!aligned(out_u64, 8)) return DIT_EALIGN;
  if (dit_status s = check_device()) return s;
  (void)hipGetLastError();
  return launched(ditq::launch_mfma_probe(workgroups, iters, static_cast<unsigned long long*>(out_u64),
                                          static_cast<hipStream_t>(stream)));
}

const char* dit_last_error(void) { return g_last_error; }

const char* dit_status_str(dit_status status) {
  switch (raw(status)) {
    case DIT_OK: return "ok";
    case DIT_EINVAL: return "invalid argument";
    case DIT_EUNSUPPORTED: return "unsupported shape or combination";
    case DIT_EALIGN: return "misaligned pointer or leading dimension";
    case DIT_EDEVICE: return "no usable gfx950 device or launch failure";
  }
  return "unknown status";
}

}  // extern "C"
