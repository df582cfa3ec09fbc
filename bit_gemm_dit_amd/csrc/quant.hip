// On-the-fly activation quantizers (gfx950).
//
// FP4: bf16 [M, K] -> E2M1 codes + E8M0 block scales, K-panel-major.  Activation
// statistics change from one diffusion iteration to the next, so the scales are
// computed from the data on every call rather than calibrated once (page
// "Versnellende diffusiemodellen met TheStage AI", section on acceleration and
// compression); the 4-bit float format is that of page "How fal made Ideogram V4
// 6x faster", paragraph 2.
// FP8: bf16 [M, K] -> E4M3 codes (K-panel-major) + fp32 row scales [M] (page "WaveSpeedAI
// X DataCrunch", engine list: FP8 mixed precision).
// MXFP8: bf16 [M, K] -> E4M3 codes (the FP8 code layout) + E8M0 block-32 scales (the
// FP4 scale layout), scales computed per call like the FP4 path's.
// NVFP4: bf16 [M, K] -> E2M1 codes (the FP4 code layout) + E4M3 block-16 scales + one
// fp32 tensor scale (the 4-bit format page "How fal made Ideogram V4 6x faster"
// names, paragraph 2), in three launches: per-workgroup maxima, the tensor maximum,
// then the quantizer.
//
// All kernels are HBM-bound streams: 2 bytes read per element, 0.5 + 1/32 (FP4),
// 1 (FP8) or 1 + 1/32 (MXFP8) bytes written.  Outputs are K-panel-major
// (include/ditq.h): the GEMM then copies each 64-byte-per-token panel slice of a
// token tile as one contiguous run.
#include <atomic>
#include <type_traits>

#include "common.hpp"

namespace ditq {
namespace {

// FP8 row quantizer, rows whose largest magnitude is at least 2^-60 (bf16 bits
// 0x2180): x / s from one reciprocal per row and one correction, q0 = fl32(|x| * r)
// with r = fl32(1 / s), then q0 + (|x| - q0 s) r with the residual exact in an FMA,
// the sign restored from x.  An exhaustive check over every bf16 amax >= 2^-60 and
// every bf16 x with |x| <= amax (tests/csrc/fp8_row_division_check.c) finds it equal to
// the IEEE quotient fl32(x / s) bit for bit wherever |x / s| >= 2^-10, and below that
// of magnitude <= 2^-10 with the sign of x, so both round to the same signed E4M3 zero:
// the codes are those of the IEEE division.  Rows with a smaller maximum keep the IEEE
// division (the residual could fall below fp32's normal range).  Four VALU operations
// per element instead of the division's sequence.
constexpr uint32_t kFp8RcpAmaxMin = 0x2180u;
__device__ inline float fp8_quotient_rcp(float x, float s, float r) {
  const float ax = __builtin_fabsf(x);
  const float q0 = ax * r;
  return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, s, ax), r, q0), x);
}
// fp8_encode4 with the quotient above: four bf16 values -> four E4M3 codes (byte i =
// element i), the same clamp and conversion.
__device__ inline uint32_t fp8_encode4_rcp(uint32_t w0, uint32_t w1, float s, float r) {
  float a = fp8_quotient_rcp(bf16_lo(w0), s, r), b = fp8_quotient_rcp(bf16_hi(w0), s, r);
  float c = fp8_quotient_rcp(bf16_lo(w1), s, r), d = fp8_quotient_rcp(bf16_hi(w1), s, r);
  a = fmaxf(fminf(a, 448.0f), -448.0f);
  b = fmaxf(fminf(b, 448.0f), -448.0f);
  c = fmaxf(fminf(c, 448.0f), -448.0f);
  d = fmaxf(fminf(d, 448.0f), -448.0f);
  int q = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  q = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, q, true);
  return (uint32_t)q;
}

// DPP quad permutations: xor 1 = [1,0,3,2], xor 2 = [2,3,0,1].
constexpr int kQuadXor1 = 0xB1;
constexpr int kQuadXor2 = 0x4E;

// DPP quad permutation that gives every lane of a quad the value of quad lane i.
constexpr int quad_bcast(int i) { return i | (i << 2) | (i << 4) | (i << 6); }

// One workgroup of 128 threads per (block of 8 tokens, 128-element K panel).  Thread
// t handles 8 consecutive elements (16 bytes of bf16) of token t/16; the four threads
// of a DPP quad cover one 32-element block and agree on its scale.  The workgroup
// writes its tokens' panel rows as whole contiguous runs: 8 x 64 code bytes (each
// quad leader stores its quad's 16 bytes) and 8 x 4 scale bytes (the first lane of
// each token's 16 stores the token's four).  Rows past M are skipped, uniformly over
// a token's 16 lanes.  Small workgroups with one load per thread measured fastest
// (same-box A/B, outputs identical, 4608 x 3072: 7.3 us back to back against 7.6 with
// 16 tokens per 256 threads, 8.0 with 32 tokens per 256 threads in two passes, and
// 8.4-9.7 with 2 or 4 panels per workgroup).
constexpr int kQ4Threads = 128;
constexpr int kQ4Tokens = kQ4Threads / 16;
__global__ __launch_bounds__(kQ4Threads) void quant_fp4_kernel(const uint16_t* __restrict__ x, int M, int ldx,
                                                               int panels, uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales) {
  const int s = blockIdx.x % panels, blk = blockIdx.x / panels;
  const int t = threadIdx.x, chunk = t & 15, row0 = t & 48;     // row0: the token's first lane in its wave
  const int tok = blk * kQ4Tokens + (t >> 4);
  if (tok >= M) return;
  const v4i v = *reinterpret_cast<const v4i*>(x + (size_t)tok * ldx + s * 128 + chunk * 8);
  uint32_t m = absmax8(v);
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kQuadXor1, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kQuadXor2, 0xF, 0xF, false));
  const uint32_t byte = fp4_scale_byte(m);
  const uint32_t q = fp4_encode8(v, byte);
  const uint32_t q1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q, quad_bcast(1), 0xF, 0xF, false);
  const uint32_t q2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q, quad_bcast(2), 0xF, 0xF, false);
  const uint32_t q3 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q, quad_bcast(3), 0xF, 0xF, false);
  const uint32_t word = byte | ((uint32_t)__shfl((int)byte, row0 + 4, 64) << 8) |
                        ((uint32_t)__shfl((int)byte, row0 + 8, 64) << 16) |
                        ((uint32_t)__shfl((int)byte, row0 + 12, 64) << 24);
  const size_t prow = (size_t)s * M + tok;                        // panel-major row index
  if ((chunk & 3) == 0)
    *reinterpret_cast<v4i*>(codes + prow * 64 + 4 * chunk) = v4i{(int)q, (int)q1, (int)q2, (int)q3};
  if (chunk == 0) *reinterpret_cast<uint32_t*>(scales + prow * 4) = word;
}

// MXFP8: the FP4 kernel's workgroup and quad structure with E4M3 elements: 128
// threads per (8 tokens, 128-element K panel s), thread t on chunk c = t % 16
// (elements 8c .. 8c+7 of the panel) of token t / 16.  The chunk's 8 codes go to
// 64-element code panel 2s + c/8 at byte 8 (c % 8) of the token's 64-byte panel row;
// the token's four block scales of the panel go out as one 4-byte word (the first lane
// of the token's 16), like the FP4 scales.  Same-box A/B against a grid-stride form
// with 256-thread workgroups that stored one scale byte per quad, codes and scales
// identical: 8.95 -> 8.29 us back to back at 4608 x 3072 (0.60 -> 0.65 of HBM).
__global__ __launch_bounds__(kQ4Threads) void quant_mx8_kernel(const uint16_t* __restrict__ x, int M, int ldx,
                                                               int panels, uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales) {
  const int s = blockIdx.x % panels, blk = blockIdx.x / panels;
  const int t = threadIdx.x, chunk = t & 15, row0 = t & 48;     // row0: the token's first lane in its wave
  const int tok = blk * kQ4Tokens + (t >> 4);
  if (tok >= M) return;
  const v4i v = *reinterpret_cast<const v4i*>(x + (size_t)tok * ldx + s * 128 + chunk * 8);
  uint32_t m = absmax8(v);
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kQuadXor1, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kQuadXor2, 0xF, 0xF, false));
  const uint32_t byte = mx8_scale_byte(m);
  uint2 q;
  q.x = mx8_encode4((uint32_t)v.x, (uint32_t)v.y, byte);
  q.y = mx8_encode4((uint32_t)v.z, (uint32_t)v.w, byte);
  const size_t crow = (size_t)(2 * s + (chunk >> 3)) * M + tok;   // code panel-major row index
  *reinterpret_cast<uint2*>(codes + crow * 64 + 8 * (chunk & 7)) = q;
  const uint32_t word = byte | ((uint32_t)__shfl((int)byte, row0 + 4, 64) << 8) |
                        ((uint32_t)__shfl((int)byte, row0 + 8, 64) << 16) |
                        ((uint32_t)__shfl((int)byte, row0 + 12, 64) << 24);
  if (chunk == 0) *reinterpret_cast<uint32_t*>(scales + ((size_t)s * M + tok) * 4) = word;
}

// Maximum of the 256 lanes' values of a workgroup (waves, then LDS), valid in thread 0.
__device__ inline uint32_t block_max256(uint32_t m, uint32_t* wave_max) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  return max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
}

// Tensor maximum, in two launches and without atomics: one thread per 8 elements,
// grid-stride over at most kAmaxBlocks workgroups, each leaving its maximum in
// partial[workgroup]; then one workgroup reduces those into the slot.  (bf16
// magnitude bit patterns order like their values, so the unsigned maximum is the
// maximum.)  Every workgroup merging into the one slot with an atomic maximum
// measured slower: those atomics are serialised on one address.
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ x, int ld, uint32_t total,
                                                   uint32_t per_row, uint32_t* partial) {
  __shared__ uint32_t wave_max[4];
  uint32_t m = 0;
  const uint32_t stride = gridDim.x * 256u;
  // eight loads in flight per thread and pass: same-box A/B of the whole NVFP4
  // quantizer (this pass, the reduction, the quantizer) at 4608 x 3072, outputs
  // identical: 19.77 us with one load per pass, 18.85 with four, 18.66 with eight.
  // (Moving the quantizer itself to 128-thread workgroups of 8 tokens, as for FP4 and
  // MXFP8, measured no faster: its per-element division dominates.)
  constexpr int kU = 8;
  for (uint32_t c = blockIdx.x * 256u + threadIdx.x; c < total; c += kU * stride) {
    v4i v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t cc = c + u * stride;
      v[u] = v4i{0, 0, 0, 0};
      if (cc < total) {
        const uint32_t row = cc / per_row, col = cc - row * per_row;
        v[u] = *reinterpret_cast<const v4i*>(x + (size_t)row * ld + (size_t)col * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) m = max(m, absmax8(v[u]));
  }
  m = block_max256(m, wave_max);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

__global__ __launch_bounds__(256) void amax_final_kernel(const uint32_t* __restrict__ partial, uint32_t n,
                                                         uint32_t* slot) {
  __shared__ uint32_t wave_max[4];
  uint32_t m = 0;
  for (uint32_t i = threadIdx.x; i < n; i += 256u) m = max(m, partial[i]);
  m = block_max256(m, wave_max);
  if (threadIdx.x == 0) slot[0] = m;
}

// NVFP4: one lane per 8 elements as in the FP4 kernel, in a grid-stride loop over
// 256-thread workgroups; a block of 16 is one lane pair (DPP xor 1).
// Chunk `col` (8 elements) goes to the FP4 code position; its block (col/2) scale to
// byte (col/2) % 8 of the token's 8-byte row of 128-element panel col/16.
__global__ __launch_bounds__(256) void quant_nv4_kernel(const uint16_t* __restrict__ x, int M, int ldx,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, uint32_t total,
                                                        uint32_t per_row, const uint32_t* amax_slot,
                                                        float* tensor_scale) {
  const float st = nv4_tensor_scale(*amax_slot);
  const float six_st = 6.0f * st;
  if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = st;
  const uint32_t stride = gridDim.x * 256u;
  for (uint32_t c = blockIdx.x * 256u + threadIdx.x; c < total; c += stride) {
    const uint32_t row = c / per_row, col = c - row * per_row;
    const v4i v = *reinterpret_cast<const v4i*>(x + (size_t)row * ldx + (size_t)col * 8);
    uint32_t m = absmax8(v);
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kQuadXor1, 0xF, 0xF, false));
    const uint32_t sb = nv4_scale_code(__uint_as_float(m << 16) / six_st);
    const float denom = __builtin_amdgcn_cvt_f32_fp8((int)sb, 0) * st;
    const size_t prow = (size_t)(col >> 4) * M + row;
    *reinterpret_cast<uint32_t*>(codes + prow * 64 + 4 * (col & 15)) = nv4_encode8(v, denom);
    if ((threadIdx.x & 1) == 0) scales[prow * 8 + ((col >> 1) & 7)] = (uint8_t)sb;
  }
}

// One wave per row.  Rows up to kMaxCached*512 elements stay in registers between
// the amax pass and the encode pass; longer rows are read twice.
constexpr int kMaxCached = 16;

template <bool CACHED>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                        int ldx, uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;                                   // uniform per wave
  const uint16_t* xr = x + (size_t)row * ldx;
  // element k lands in K panel k/64 (64 elements per panel), byte k%64 of the token's panel row
  auto dst = [&](int k) { return codes + ((size_t)(k >> 6) * M + row) * 64 + (k & 63); };
  const int nch = (K + 511) / 512;
  uint32_t m = 0;
  v4i cache[CACHED ? kMaxCached : 1];
  if (CACHED) {
#pragma unroll
    for (int i = 0; i < kMaxCached; ++i) {
      const int k = i * 512 + lane * 8;
      if (i < nch && k < K) {
        cache[i] = *reinterpret_cast<const v4i*>(xr + k);
        m = max(m, absmax8(cache[i]));
      }
    }
  } else {
    for (int i = 0; i < nch; ++i) {
      const int k = i * 512 + lane * 8;
      if (k < K) m = max(m, absmax8(*reinterpret_cast<const v4i*>(xr + k)));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  const float s = fp8_row_scale(m);
  if (lane == 0) scales[row] = s;
  const float r = 1.0f / s;
  auto encode_row = [&](auto rcp_c) __attribute__((always_inline)) {
    constexpr bool RCP = decltype(rcp_c)::value;
    auto enc = [&](const v4i& v) __attribute__((always_inline)) {
      uint2 q;
      if constexpr (RCP) {
        q.x = fp8_encode4_rcp((uint32_t)v.x, (uint32_t)v.y, s, r);
        q.y = fp8_encode4_rcp((uint32_t)v.z, (uint32_t)v.w, s, r);
      } else {
        q.x = fp8_encode4((uint32_t)v.x, (uint32_t)v.y, s);
        q.y = fp8_encode4((uint32_t)v.z, (uint32_t)v.w, s);
      }
      return q;
    };
    if (CACHED) {
#pragma unroll
      for (int i = 0; i < kMaxCached; ++i) {
        const int k = i * 512 + lane * 8;
        if (i < nch && k < K) *reinterpret_cast<uint2*>(dst(k)) = enc(cache[i]);
      }
    } else {
      for (int i = 0; i < nch; ++i) {
        const int k = i * 512 + lane * 8;
        if (k < K) *reinterpret_cast<uint2*>(dst(k)) = enc(*reinterpret_cast<const v4i*>(xr + k));
      }
    }
  };
  // m is the row's maximum in every lane, so the choice is uniform over the wave
  if (m >= kFp8RcpAmaxMin) encode_row(std::true_type{});
  else encode_row(std::false_type{});
}

}  // namespace

hipError_t launch_quant_fp4(const uint16_t* x, int M, int K, int ldx, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream) {
  const int panels = K / 128;
  const uint32_t blocks = (uint32_t)((M + kQ4Tokens - 1) / kQ4Tokens) * (uint32_t)panels;
  hipLaunchKernelGGL(quant_fp4_kernel, dim3(blocks), dim3(kQ4Threads), 0, stream, x, M, ldx, panels, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_mx8(const uint16_t* x, int M, int K, int ldx, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream) {
  const int panels = K / 128;
  const uint32_t blocks = (uint32_t)((M + kQ4Tokens - 1) / kQ4Tokens) * (uint32_t)panels;
  hipLaunchKernelGGL(quant_mx8_kernel, dim3(blocks), dim3(kQ4Threads), 0, stream, x, M, ldx, panels, codes, scales);
  return hipGetLastError();
}

hipError_t launch_amax_bf16(const uint16_t* x, int R, int cols, int ld, uint32_t* slot, uint32_t* partial,
                            hipStream_t stream) {
  const uint32_t per_row = (uint32_t)cols / 8;
  const uint32_t total = (uint32_t)R * per_row;
  uint32_t blocks = (total + 255) / 256;
  if (blocks > kAmaxBlocks) blocks = kAmaxBlocks;         // two workgroups per CU, grid-stride beyond
  hipLaunchKernelGGL(amax_kernel, dim3(blocks), dim3(256), 0, stream, x, ld, total, per_row, partial);
  hipLaunchKernelGGL(amax_final_kernel, dim3(1), dim3(256), 0, stream, partial, blocks, slot);
  return hipGetLastError();
}

hipError_t launch_quant_nv4(const uint16_t* x, int M, int K, int ldx, uint8_t* codes, uint8_t* scales,
                            uint32_t* work, hipStream_t stream) {
  uint32_t* slot = reinterpret_cast<uint32_t*>(scales + nv4_act_tail(M, K));
  // work: the tensor-maximum slot and the per-workgroup maxima; by default the
  // scale buffer's own tail (slot, then the maxima after the 16-byte tail)
  uint32_t* amax = work ? work : slot;
  uint32_t* partial = work ? work + 1 : slot + kNvTailBytes / 4;
  if (hipError_t e = launch_amax_bf16(x, M, K, ldx, amax, partial, stream)) return e;
  const uint32_t per_row = (uint32_t)K / 8;
  const uint32_t total = (uint32_t)M * per_row;
  uint32_t blocks = (total + 255) / 256;
  const uint32_t cap = 256u * 32u;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(quant_nv4_kernel, dim3(blocks), dim3(256), 0, stream, x, M, ldx, codes, scales, total,
                     per_row, amax, reinterpret_cast<float*>(slot + 1));
  return hipGetLastError();
}

// Work space of the allocation-free NVFP4 quantizer: the tensor-maximum slot and the
// kAmaxBlocks per-workgroup maxima, 2052 bytes whatever M and K.  Each device holds
// its own copy until the process ends; every call on that device shares it, so calls
// that overlap on one device race.  Nothing in it needs clearing: every call writes
// each entry it reads first.
static __device__ __align__(256) uint32_t scratch[1 + kAmaxBlocks];

// Device address of `scratch` on the current device, looked up once per device
// (the host-side name is only a stand-in: a kernel must be given this address).
static hipError_t scratch_address(uint32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<uint32_t*> addr[kMaxDevices];
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uint32_t* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch))) return e;
    p = static_cast<uint32_t*>(q);
    addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_quant_nv4_static(const uint16_t* x, int M, int K, int ldx, uint8_t* codes, uint8_t* scales,
                                   hipStream_t stream) {
  uint32_t* work = nullptr;
  if (hipError_t e = scratch_address(&work)) return e;
  return launch_quant_nv4(x, M, K, ldx, codes, scales, work, stream);
}

hipError_t launch_quant_fp8(const uint16_t* x, int M, int K, int ldx, uint8_t* codes, float* scales,
                            hipStream_t stream) {
  const dim3 grid((M + 3) / 4);
  if (K <= kMaxCached * 512)
    hipLaunchKernelGGL(quant_fp8_kernel<true>, grid, dim3(256), 0, stream, x, M, K, ldx, codes, scales);
  else
    hipLaunchKernelGGL(quant_fp8_kernel<false>, grid, dim3(256), 0, stream, x, M, K, ldx, codes, scales);
  return hipGetLastError();
}

}  // namespace ditq
