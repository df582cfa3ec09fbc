// Kernels that measure the fused path rather than compute it.
//
// * gated_silu_kernel: the gated-SiLU epilogue as a separate pass over a bf16 GEMM
//   output C = [gate | up] (the unfused form: C is written to HBM by an identity
//   GEMM and read back here).  Timing it next to the fused GEMM gives the saving of
//   applying the small op before the single store (page "How fal made Ideogram V4
//   6x faster", paragraph 3; the split-and-multiply op: paragraph 4).  The same
//   SiLU arithmetic as the fused epilogue, on C rounded to bf16.
// * mfma_probe_kernel: FP4 scaled MFMAs on register operands only, no memory
//   traffic, so the matrix cores' sustained rate at the clock the chip holds under
//   that load can be set beside the spec peak.
#include "common.hpp"

namespace ditq {
namespace {

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ inline uint32_t pack2_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, b2));
}

// x / (1 + e^-x) with the hardware exp2 and reciprocal, as in the fused epilogue
__device__ inline float silu_f32(float x) {
  const float e = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// One thread per 8 output columns: 16 bytes of gate, 16 bytes of up, 16 bytes out.
__global__ __launch_bounds__(256) void gated_silu_kernel(const uint16_t* __restrict__ c, int ldc, int half,
                                                         uint16_t* __restrict__ out, int ldo, uint32_t total,
                                                         uint32_t per_row) {
  const uint32_t stride = gridDim.x * 256u;
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < total; i += stride) {
    const uint32_t row = i / per_row, col = 8u * (i - row * per_row);
    const uint16_t* cr = c + (size_t)row * ldc + col;
    const v4i g = *reinterpret_cast<const v4i*>(cr);
    const v4i u = *reinterpret_cast<const v4i*>(cr + half);
    v4i o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t gw = (uint32_t)g[k], uw = (uint32_t)u[k];
      const float g0 = bf16_to_f32(gw & 0xFFFFu), g1 = bf16_to_f32(gw >> 16);
      const float u0 = bf16_to_f32(uw & 0xFFFFu), u1 = bf16_to_f32(uw >> 16);
      o[k] = (int)pack2_bf16(silu_f32(g0) * u0, silu_f32(g1) * u1);
    }
    *reinterpret_cast<v4i*>(out + (size_t)row * ldo + col) = o;
  }
}

// Eight independent 32x32x64 FP4 MFMAs per iteration and wave (eight accumulators,
// so consecutive MFMAs never wait on each other), operands in registers.  Wave 0 of
// each workgroup records s_memtime around its loop; every wave folds its sums into a
// checksum so that nothing is optimised away.
constexpr int kProbeAcc = 8;

__global__ __launch_bounds__(256, 1) void mfma_probe_kernel(int iters, unsigned long long* out) {
  const int lane = threadIdx.x & 63;
  v8i a = {lane, lane + 1, lane + 2, lane + 3, 0, 0, 0, 0};
  v8i b = {lane ^ 5, lane ^ 6, lane ^ 7, lane ^ 8, 0, 0, 0, 0};
  v16f acc[kProbeAcc];
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j) acc[j] = v16f{};
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 4, 4, 0, 127, 0, 127);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  s += __shfl_xor(s, 32);
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = t1 - t0;
    out[2 * blockIdx.x + 1] = (unsigned long long)__float_as_uint(s);
  }
}

}  // namespace

hipError_t launch_gated_silu(const uint16_t* c, int M, int N, int ldc, uint16_t* out, int ldo,
                             hipStream_t stream) {
  const uint32_t per_row = (uint32_t)(N / 2) / 8;
  const uint32_t total = (uint32_t)M * per_row;
  uint32_t blocks = (total + 255) / 256;
  const uint32_t cap = 256u * 16u;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(gated_silu_kernel, dim3(blocks), dim3(256), 0, stream, c, ldc, N / 2, out, ldo, total,
                     per_row);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int workgroups, int iters, unsigned long long* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(256), 0, stream, iters, out);
  return hipGetLastError();
}

}  // namespace ditq
