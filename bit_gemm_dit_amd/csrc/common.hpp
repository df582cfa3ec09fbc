// Shared device/host definitions of the fused low-bit linear layer (gfx950).
//
// Blob layout constants, vector types and the FP4 / FP8 / MXFP8 element encoders
// used by both the activation quantizer and the weight packer.  The encoders follow
// the quantization rules documented in include/ditq.h (FP4, per 32-element block:
// E8M0 scale = 2^(floor(log2 amax) - 2), element = RNE_E2M1(x / scale); FP8:
// RNE_E4M3 of x / s with s = amax / 448; MXFP8, per 32-element block: E8M0 scale
// = 2^(floor(log2 amax) - 8), element = RNE_E4M3(x / scale)), the formats of page
// "How fal made Ideogram V4 6x faster" (paragraph 2, a 4-bit float format) and
// page "WaveSpeedAI X DataCrunch" (engine list, FP8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ditq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

enum { FMT_FP4 = 1, FMT_FP8 = 2, FMT_MX8 = 3, FMT_NV4 = 4 };
enum { EPI_IDENTITY = 0, EPI_GATED_SILU = 1, EPI_QK_RMSNORM = 2, EPI_GELU_TANH = 3, EPI_GATE_RESIDUAL = 4 };

// ---------------------------------------------------------------- blob layout
constexpr uint32_t kBlobMagic = 0x51544944u;   // "DITQ"
constexpr uint32_t kBlobVersion = 2;
constexpr int kHeaderBytes = 256;
constexpr int kRowPad = 256;                   // packed rows are padded to a multiple of this

__host__ __device__ inline int padded_rows(int N) { return (N + kRowPad - 1) / kRowPad * kRowPad; }
constexpr int kNvTensorScaleOff = 56;          // NVFP4 blob: fp32 tensor scale in the header
constexpr int kNvAmaxOff = 60;                 // ... and the packer's tensor-maximum slot

__host__ __device__ constexpr bool is_fp4_codes(int fmt) { return fmt == FMT_FP4 || fmt == FMT_NV4; }
__host__ __device__ inline size_t blob_code_bytes(int fmt, int Np, int K) {
  return is_fp4_codes(fmt) ? (size_t)Np * K / 2 : (size_t)Np * K;
}
__host__ __device__ inline size_t blob_scale_bytes(int fmt, int Np, int K) {
  return fmt == FMT_FP8 ? (size_t)Np * 4 : fmt == FMT_NV4 ? (size_t)Np * K / 16 : (size_t)Np * K / 32;
}
// NVFP4 activation scales: M*K/16 block scale bytes, then a 16-byte tail holding the
// tensor-maximum slot (u32) and the fp32 tensor scale, then the per-workgroup maxima
// of the tensor-maximum pass (kAmaxBlocks u32).
constexpr uint32_t kAmaxBlocks = 512;
constexpr int kNvTailBytes = 16;
constexpr int kNvPartialBytes = 4 * kAmaxBlocks;
__host__ __device__ inline size_t nv4_act_tail(int M, int K) { return (size_t)M * K / 16; }
__host__ __device__ inline size_t blob_scales_offset(int fmt, int Np, int K) {
  return kHeaderBytes + blob_code_bytes(fmt, Np, K);
}
__host__ __device__ inline size_t blob_total_bytes(int fmt, int Np, int K) {
  return blob_scales_offset(fmt, Np, K) + blob_scale_bytes(fmt, Np, K);
}
// Logical weight row stored at packed row p, or -1 for padding.  For gated-SiLU
// each 64-row group holds 32 gate rows followed by their 32 up rows.
__host__ __device__ inline int packed_row_source(int epi, int N, int p) {
  if (p >= N) return -1;
  if (epi != EPI_GATED_SILU) return p;
  const int P = p >> 6, i = p & 63;
  return i < 32 ? 32 * P + i : N / 2 + 32 * P + (i - 32);
}

// ---------------------------------------------------------------- FP4 encoding
// E8M0 scale byte from the largest bf16 magnitude of a block (bit pattern with
// the sign cleared).  Magnitude order equals integer order for finite bf16, and
// floor(log2 amax) - 2 + 127 clamped at 0 reduces to max(exponent field - 2, 0):
// subnormal maxima have exponent field 0 and clamp to 0 as well.
__device__ inline uint32_t fp4_scale_byte(uint32_t amax_bits) {
  const uint32_t ex = amax_bits >> 7;
  return ex > 2 ? ex - 2 : 0;
}

// Double a bf16 magnitude/sign pattern exactly (only used on blocks whose maximum
// has an exponent field <= 2, so no overflow): subnormals shift left, which also
// carries correctly into the smallest normal binade; normals add one to the exponent.
__device__ inline uint32_t bf16_double_bits(uint32_t b) {
  const uint32_t s = b & 0x8000u, m = b & 0x7FFFu;
  return s | ((m >> 7) == 0 ? (m << 1) : (m + 0x80u));
}
__device__ inline uint32_t bf16x2_double(uint32_t w) {
  return bf16_double_bits(w & 0xFFFFu) | (bf16_double_bits(w >> 16) << 16);
}

// 8 bf16 values (one uint4) -> 8 E2M1 codes (one dword, element 2j in the low
// nibble of byte j) for scale byte `byte`.  The hardware conversion computes
// RNE_E2M1(x / scale) with saturation at 6 and the sign kept; it takes the scale
// as an fp32 power of two.  Byte 0 would need the subnormal float 2^-127, so
// there the values are doubled exactly and divided by 2^-126 instead.
__device__ inline uint32_t fp4_encode8(v4i v, uint32_t byte) {
  uint32_t w0 = (uint32_t)v.x, w1 = (uint32_t)v.y, w2 = (uint32_t)v.z, w3 = (uint32_t)v.w;
  uint32_t sbits = byte << 23;
  if (byte == 0) {
    w0 = bf16x2_double(w0); w1 = bf16x2_double(w1); w2 = bf16x2_double(w2); w3 = bf16x2_double(w3);
    sbits = 1u << 23;
  }
  const float scale = __uint_as_float(sbits);
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w0), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w1), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w2), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w3), scale, 3);
  return r;
}

__device__ inline uint32_t bf16x2_absmax(uint32_t w) {
  const uint32_t a = w & 0x7FFFu, b = (w >> 16) & 0x7FFFu;
  return a > b ? a : b;
}
__device__ inline uint32_t absmax8(v4i v) {
  uint32_t m = bf16x2_absmax((uint32_t)v.x);
  m = max(m, bf16x2_absmax((uint32_t)v.y));
  m = max(m, bf16x2_absmax((uint32_t)v.z));
  m = max(m, bf16x2_absmax((uint32_t)v.w));
  return m;
}

// ---------------------------------------------------------------- FP8 encoding
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Row scale s = fl32(amax / 448) (IEEE division), 1 for an all-zero row.
__device__ inline float fp8_row_scale(uint32_t amax_bits) {
  const float amax = __uint_as_float(amax_bits << 16);
  return amax_bits == 0 ? 1.0f : amax / 448.0f;
}

// Four bf16 values -> four E4M3 codes (byte i = element i): q = RNE_E4M3(fl32(x / s)).
// |x / s| <= 448 * (1 + 2^-23) by construction; the clamp keeps values in the
// hardware conversion's saturating range without changing any rounding.
__device__ inline uint32_t fp8_encode4(uint32_t w0, uint32_t w1, float s) {
  float a = bf16_lo(w0) / s, b = bf16_hi(w0) / s, c = bf16_lo(w1) / s, d = bf16_hi(w1) / s;
  a = fmaxf(fminf(a, 448.0f), -448.0f);
  b = fmaxf(fminf(b, 448.0f), -448.0f);
  c = fmaxf(fminf(c, 448.0f), -448.0f);
  d = fmaxf(fminf(d, 448.0f), -448.0f);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

// ---------------------------------------------------------------- MXFP8 encoding
// E8M0 scale byte of an MXFP8 block from its largest bf16 magnitude (sign cleared):
// floor(log2 amax) - 8 + 127 clamped at 0 is max(exponent field - 8, 0); subnormal
// maxima (exponent field 0) clamp to 0 as well.  At most 246 for finite bf16.
__device__ inline uint32_t mx8_scale_byte(uint32_t amax_bits) {
  const uint32_t ex = amax_bits >> 7;
  return ex > 8 ? ex - 8 : 0;
}

// Four bf16 values -> four E4M3 codes (byte i = element i) for scale byte `byte`:
// RNE_E4M3(x * 2^(127 - byte)).  The factor is a normal fp32 power of two for every
// byte <= 246, so the product is exact down to fp32's normal range; smaller
// products lie far below E4M3's smallest rounding threshold (2^-10) and encode as a
// signed zero either way.  The clamp is the saturation at 448.
__device__ inline uint32_t mx8_encode4(uint32_t w0, uint32_t w1, uint32_t byte) {
  const float f = __uint_as_float((254u - byte) << 23);
  float a = bf16_lo(w0) * f, b = bf16_hi(w0) * f, c = bf16_lo(w1) * f, d = bf16_hi(w1) * f;
  a = fmaxf(fminf(a, 448.0f), -448.0f);
  b = fmaxf(fminf(b, 448.0f), -448.0f);
  c = fmaxf(fminf(c, 448.0f), -448.0f);
  d = fmaxf(fminf(d, 448.0f), -448.0f);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

// ---------------------------------------------------------------- NVFP4 encoding
// Two levels of scaling (every step IEEE fp32): s_t = fl32(amax_tensor / 2688) (1 for
// a zero tensor); per 16-element block s_b = RNE_E4M3(min(fl32(amax_b / fl32(6 s_t)),
// 448)); elements RNE_E2M1(fl32(x / fl32(dec(s_b) s_t))), saturating at 6.
__device__ inline float nv4_tensor_scale(uint32_t amax_bits) {
  return amax_bits == 0 ? 1.0f : __uint_as_float(amax_bits << 16) / 2688.0f;
}
// E4M3 code of a non-negative block ratio d (round to nearest even, saturating).
__device__ inline uint32_t nv4_scale_code(float d) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(d, 448.0f), 0.0f, 0, false) & 0xFFu;
}
// Eight bf16 values (one uint4) -> eight E2M1 codes (one dword, element 2j in the low
// nibble of byte j), divided by `denom` = fl32(dec(s_b) * s_t).  The division is the
// IEEE fp32 one; the conversion (scale 1) rounds to nearest even, saturates at 6 and
// keeps the sign.  denom = 0 (an all-zero block scale) gives signed zeros.
__device__ inline uint32_t nv4_encode8(v4i v, float denom) {
  float y[8];
  const uint32_t w[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf16_lo(w[i]), hi = bf16_hi(w[i]);
    y[2 * i] = denom == 0.0f ? lo * 0.0f : lo / denom;
    y[2 * i + 1] = denom == 0.0f ? hi * 0.0f : hi / denom;
  }
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[0], y[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[2], y[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[4], y[5], 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[6], y[7], 1.0f, 3);
  return r;
}

// ---------------------------------------------------------------- buffer resources
// Raw buffer descriptors: loads past num_records bytes return zeros, which
// clips ragged tiles without branches.
constexpr int kBufferFlags = 0x00020000;
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

// ---------------------------------------------------------------- launchers (host)
struct RmsArgs {
  int head_dim;
  int n_heads;
  const float* gamma_q;
  const float* gamma_k;
  float eps;
};
struct ResidualArgs {
  const uint16_t* residual;   // bf16 [M][ldr]; may be the output itself
  int ldr;
  const float* gate;          // fp32 [ceil(M / rows_per_gate)][N]
  int rows_per_gate;
};

hipError_t launch_quant_fp4(const uint16_t* x, int M, int K, int ldx, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream);
hipError_t launch_quant_fp8(const uint16_t* x, int M, int K, int ldx, uint8_t* codes, float* scales,
                            hipStream_t stream);
hipError_t launch_quant_mx8(const uint16_t* x, int M, int K, int ldx, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream);
// scales: M*K/16 block scale bytes plus the tail (nv4_act_tail, kNvTailBytes + kNvPartialBytes).
// work: 1 + kAmaxBlocks u32 of work space for the tensor maximum, or null to use the
// scale buffer's tail for it.
hipError_t launch_quant_nv4(const uint16_t* x, int M, int K, int ldx, uint8_t* codes, uint8_t* scales,
                            uint32_t* work, hipStream_t stream);
// The same with the library's static per-device work space (quant.hip `scratch`): the
// scale buffer then needs only M*K/16 + kNvTailBytes bytes.  No allocation.
hipError_t launch_quant_nv4_static(const uint16_t* x, int M, int K, int ldx, uint8_t* codes, uint8_t* scales,
                                   hipStream_t stream);
// Largest bf16 magnitude (bit pattern) of x [R][ld] (first `cols` columns), written to
// *slot; `partial` is work space for kAmaxBlocks u32 (the per-workgroup maxima).
hipError_t launch_amax_bf16(const uint16_t* x, int R, int cols, int ld, uint32_t* slot, uint32_t* partial,
                            hipStream_t stream);
hipError_t launch_pack(int fmt, int epi, const uint16_t* w, int N, int K, int ldw, uint8_t* blob,
                       hipStream_t stream);
// Fused GEMM + epilogue in any format.  a_scales: FP4 / MXFP8 E8M0 bytes, FP8 fp32
// row scales.  rms: non-null exactly for EPI_QK_RMSNORM; gr: exactly for
// EPI_GATE_RESIDUAL.  q_codes / q_scales (FP4 only): optional FP4 quantization of
// the output (null: none); out may be null when q_codes is set.  out_f32 (debug, or
// null): the fp32 values the bf16 store would round go there instead, [M][ldo] fp32.
hipError_t launch_gemm(int fmt, const uint8_t* a_codes, const void* a_scales, const uint8_t* blob, int M, int N,
                       int K, int epi, const RmsArgs* rms, const ResidualArgs* gr, uint16_t* out, int ldo,
                       uint8_t* q_codes, uint8_t* q_scales, float* out_f32, hipStream_t stream);

// measurement kernels (measure.hip)
hipError_t launch_gated_silu(const uint16_t* c, int M, int N, int ldc, uint16_t* out, int ldo,
                             hipStream_t stream);
hipError_t launch_mfma_probe(int workgroups, int iters, unsigned long long* out, hipStream_t stream);

}  // namespace ditq
