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
#include "common.hpp"

namespace ditq {
namespace {

// DPP quad permutations: xor 1 = [1,0,3,2], xor 2 = [2,3,0,1].
constexpr int kQuadXor1 = 0xB1;
constexpr int kQuadXor2 = 0x4E;

// One thread per 8 consecutive elements (16 bytes of bf16); the four threads of a
// DPP quad cover one 32-element block and agree on its scale.  Grid-stride over
// all chunks; the chunk count and the stride are multiples of 4, so quads are
// always fully active together.  Chunk `col` of a row sits in K panel col/16
// (128 elements per panel): codes at byte 4*(col%16) of the token's 64-byte panel
// row, the block scale at byte (col/4)%4 of its 4-byte panel row.
__global__ __launch_bounds__(256) void quant_fp4_kernel(const uint16_t* __restrict__ x, int M, int ldx,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, uint32_t total,
                                                        uint32_t per_row) {
  const uint32_t stride = gridDim.x * 256u;
  for (uint32_t c = blockIdx.x * 256u + threadIdx.x; c < total; c += stride) {
    const uint32_t row = c / per_row, col = c - row * per_row;
    const v4i v = *reinterpret_cast<const v4i*>(x + (size_t)row * ldx + (size_t)col * 8);
    uint32_t m = absmax8(v);
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kQuadXor1, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kQuadXor2, 0xF, 0xF, false));
    const uint32_t byte = fp4_scale_byte(m);
    const size_t prow = (size_t)(col >> 4) * M + row;              // panel-major row index
    *reinterpret_cast<uint32_t*>(codes + prow * 64 + 4 * (col & 15)) = fp4_encode8(v, byte);
    if ((threadIdx.x & 3) == 0) scales[prow * 4 + ((col >> 2) & 3)] = (uint8_t)byte;
  }
}

// MXFP8: the FP4 kernel's thread and quad structure with E4M3 elements.  Chunk
// `col` (8 elements) of a row sits in 64-element code panel col/8 at byte
// 8*(col%8) of the token's 64-byte panel row; its block scale goes to 128-element
// scale panel col/16, byte (col/4)%4 of the token's 4-byte panel row.
__global__ __launch_bounds__(256) void quant_mx8_kernel(const uint16_t* __restrict__ x, int M, int ldx,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, uint32_t total,
                                                        uint32_t per_row) {
  const uint32_t stride = gridDim.x * 256u;
  for (uint32_t c = blockIdx.x * 256u + threadIdx.x; c < total; c += stride) {
    const uint32_t row = c / per_row, col = c - row * per_row;
    const v4i v = *reinterpret_cast<const v4i*>(x + (size_t)row * ldx + (size_t)col * 8);
    uint32_t m = absmax8(v);
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kQuadXor1, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, kQuadXor2, 0xF, 0xF, false));
    const uint32_t byte = mx8_scale_byte(m);
    uint2 q;
    q.x = mx8_encode4((uint32_t)v.x, (uint32_t)v.y, byte);
    q.y = mx8_encode4((uint32_t)v.z, (uint32_t)v.w, byte);
    *reinterpret_cast<uint2*>(codes + ((size_t)(col >> 3) * M + row) * 64 + 8 * (col & 7)) = q;
    if ((threadIdx.x & 3) == 0) scales[((size_t)(col >> 4) * M + row) * 4 + ((col >> 2) & 3)] = (uint8_t)byte;
  }
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
  for (uint32_t c = blockIdx.x * 256u + threadIdx.x; c < total; c += stride) {
    const uint32_t row = c / per_row, col = c - row * per_row;
    m = max(m, absmax8(*reinterpret_cast<const v4i*>(x + (size_t)row * ld + (size_t)col * 8)));
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

// NVFP4: the FP4 kernel's structure; a block of 16 is one lane pair (DPP xor 1).
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
  if (CACHED) {
#pragma unroll
    for (int i = 0; i < kMaxCached; ++i) {
      const int k = i * 512 + lane * 8;
      if (i < nch && k < K) {
        const v4i v = cache[i];
        uint2 q;
        q.x = fp8_encode4((uint32_t)v.x, (uint32_t)v.y, s);
        q.y = fp8_encode4((uint32_t)v.z, (uint32_t)v.w, s);
        *reinterpret_cast<uint2*>(dst(k)) = q;
      }
    }
  } else {
    for (int i = 0; i < nch; ++i) {
      const int k = i * 512 + lane * 8;
      if (k < K) {
        const v4i v = *reinterpret_cast<const v4i*>(xr + k);
        uint2 q;
        q.x = fp8_encode4((uint32_t)v.x, (uint32_t)v.y, s);
        q.y = fp8_encode4((uint32_t)v.z, (uint32_t)v.w, s);
        *reinterpret_cast<uint2*>(dst(k)) = q;
      }
    }
  }
}

}  // namespace

hipError_t launch_quant_fp4(const uint16_t* x, int M, int K, int ldx, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream) {
  const uint32_t per_row = (uint32_t)K / 8;
  const uint32_t total = (uint32_t)M * per_row;
  // enough threads for one chunk each up to ~8 resident waves per SIMD; grid-stride beyond
  uint32_t blocks = (total + 255) / 256;
  const uint32_t cap = 256u * 32u;                        // 256 CUs x 32 blocks of 4 waves
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(quant_fp4_kernel, dim3(blocks), dim3(256), 0, stream, x, M, ldx, codes, scales, total,
                     per_row);
  return hipGetLastError();
}

hipError_t launch_quant_mx8(const uint16_t* x, int M, int K, int ldx, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream) {
  const uint32_t per_row = (uint32_t)K / 8;
  const uint32_t total = (uint32_t)M * per_row;
  uint32_t blocks = (total + 255) / 256;
  const uint32_t cap = 256u * 32u;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(quant_mx8_kernel, dim3(blocks), dim3(256), 0, stream, x, M, ldx, codes, scales, total,
                     per_row);
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
                            hipStream_t stream) {
  uint32_t* slot = reinterpret_cast<uint32_t*>(scales + nv4_act_tail(M, K));
  if (hipError_t e = launch_amax_bf16(x, M, K, ldx, slot, slot + kNvTailBytes / 4, stream)) return e;
  const uint32_t per_row = (uint32_t)K / 8;
  const uint32_t total = (uint32_t)M * per_row;
  uint32_t blocks = (total + 255) / 256;
  const uint32_t cap = 256u * 32u;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(quant_nv4_kernel, dim3(blocks), dim3(256), 0, stream, x, M, ldx, codes, scales, total,
                     per_row, slot, reinterpret_cast<float*>(slot + 1));
  return hipGetLastError();
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
