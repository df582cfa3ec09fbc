// Weight packer (gfx950): bf16 W [N, K] -> packed blob (layout in include/ditq.h).
//
// The codes are pre-shuffled into the MFMA operand layout: one 1 KB (FP4) or 2 KB
// (FP8, MXFP8) fragment holds, lane by lane, exactly the registers of one 32x32x64 MFMA
// operand, so the GEMM copies tiles to LDS and reads fragments with contiguous,
// conflict-free 16-byte accesses.  For gated-SiLU the rows are permuted so that
// gate row j and up row j + N/2 sit in the same lane of adjacent 32-row groups:
// "the columns of B are permuted at packing time so that each pair sits together"
// (page "How fal made Ideogram V4 6x faster", paragraph 4).  Runs once per weight.
#include "common.hpp"

namespace ditq {
namespace {

__device__ void write_header(uint8_t* blob, int fmt, int epi, int N, int K, int Np) {
  uint32_t* h = reinterpret_cast<uint32_t*>(blob);
  for (int i = 0; i < kHeaderBytes / 4; ++i) h[i] = 0;
  h[0] = kBlobMagic;
  h[1] = kBlobVersion;
  h[2] = (uint32_t)fmt;
  h[3] = (uint32_t)epi;
  h[4] = (uint32_t)N;
  h[5] = (uint32_t)K;
  h[6] = (uint32_t)Np;
  uint64_t* h64 = reinterpret_cast<uint64_t*>(blob + 32);
  h64[0] = kHeaderBytes;
  h64[1] = blob_scales_offset(fmt, Np, K);
  h64[2] = blob_total_bytes(fmt, Np, K);
}

// FP4: one thread per (fragment, lane): that lane's 32 K elements are exactly one
// E8M0 block of one weight row, so the thread computes the block scale and the 16
// code bytes on its own.
__global__ __launch_bounds__(256) void pack_fp4_kernel(const uint16_t* __restrict__ w, int N, int K,
                                                       int ldw, int epi, int Np,
                                                       uint8_t* __restrict__ blob) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  const uint32_t kc = (uint32_t)K / 64;
  const uint32_t total = (uint32_t)Np / 32 * kc * 64;
  if (t == 0) write_header(blob, FMT_FP4, epi, N, K, Np);
  if (t >= total) return;
  const uint32_t L = t & 63, frag = t >> 6;
  const uint32_t c = frag % kc, g = frag / kc;
  const int p = (int)(32 * g + (L & 31));
  const int src = packed_row_source(epi, N, p);
  v4i out = {0, 0, 0, 0};
  uint32_t byte = 0;
  if (src >= 0) {
    const v4i* wp = reinterpret_cast<const v4i*>(w + (size_t)src * ldw + 64 * c + 32 * (L >> 5));
    const v4i v0 = wp[0], v1 = wp[1], v2 = wp[2], v3 = wp[3];
    const uint32_t m = max(max(absmax8(v0), absmax8(v1)), max(absmax8(v2), absmax8(v3)));
    byte = fp4_scale_byte(m);
    out.x = (int)fp4_encode8(v0, byte);
    out.y = (int)fp4_encode8(v1, byte);
    out.z = (int)fp4_encode8(v2, byte);
    out.w = (int)fp4_encode8(v3, byte);
  }
  *reinterpret_cast<v4i*>(blob + kHeaderBytes + (size_t)frag * 1024 + 16 * L) = out;
  // scale record (s = c / 2, g), byte 2L + j with j = c % 2: block 4s + 2j + L/32 == 2c + L/32
  uint8_t* sc = blob + blob_scales_offset(FMT_FP4, Np, K);
  sc[((size_t)(c / 2) * (Np / 32) + g) * 128 + 2 * L + (c & 1)] = (uint8_t)byte;
}

// 8-bit fragments (FP8, MXFP8) hold the K order of the 32x32x64 MFMA's 8-bit
// operands: lane L's bytes 0..15 are k = 64c + 16h + (0..15) and bytes 16..31 are
// k = 64c + 32 + 16h + (0..15), h = L/32.  So the 32-element block 64c + 32j is
// split over the j-th 16-byte halves of both lane groups (whose scale the lanes of
// group j supply).

// MXFP8: one thread per (fragment, lane), as FP4; the two 16-element runs of a
// lane belong to blocks 2c and 2c + 1, and each block's maximum is shared with the
// partner lane L ^ 32 (same row) that holds the block's other run.
__global__ __launch_bounds__(256) void pack_mx8_kernel(const uint16_t* __restrict__ w, int N, int K,
                                                       int ldw, int epi, int Np,
                                                       uint8_t* __restrict__ blob) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  const uint32_t kc = (uint32_t)K / 64;
  const uint32_t total = (uint32_t)Np / 32 * kc * 64;
  if (t == 0) write_header(blob, FMT_MX8, epi, N, K, Np);
  if (t >= total) return;                                  // whole waves: total is a multiple of 64
  const uint32_t L = t & 63, frag = t >> 6, h = L >> 5;
  const uint32_t c = frag % kc, g = frag / kc;
  const int p = (int)(32 * g + (L & 31));
  const int src = packed_row_source(epi, N, p);            // the same for L and L ^ 32
  v4i a = {0, 0, 0, 0}, b = a, d = a, e = a;
  if (src >= 0) {
    const uint16_t* wr = w + (size_t)src * ldw + 64 * c + 16 * h;
    a = reinterpret_cast<const v4i*>(wr)[0];
    b = reinterpret_cast<const v4i*>(wr)[1];
    d = reinterpret_cast<const v4i*>(wr + 32)[0];
    e = reinterpret_cast<const v4i*>(wr + 32)[1];
  }
  uint32_t m0 = max(absmax8(a), absmax8(b)), m1 = max(absmax8(d), absmax8(e));
  m0 = max(m0, (uint32_t)__shfl_xor((int)m0, 32));
  m1 = max(m1, (uint32_t)__shfl_xor((int)m1, 32));
  const uint32_t byte0 = src >= 0 ? mx8_scale_byte(m0) : 0, byte1 = src >= 0 ? mx8_scale_byte(m1) : 0;
  v4i lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
  if (src >= 0) {
    lo.x = (int)mx8_encode4((uint32_t)a.x, (uint32_t)a.y, byte0);
    lo.y = (int)mx8_encode4((uint32_t)a.z, (uint32_t)a.w, byte0);
    lo.z = (int)mx8_encode4((uint32_t)b.x, (uint32_t)b.y, byte0);
    lo.w = (int)mx8_encode4((uint32_t)b.z, (uint32_t)b.w, byte0);
    hi.x = (int)mx8_encode4((uint32_t)d.x, (uint32_t)d.y, byte1);
    hi.y = (int)mx8_encode4((uint32_t)d.z, (uint32_t)d.w, byte1);
    hi.z = (int)mx8_encode4((uint32_t)e.x, (uint32_t)e.y, byte1);
    hi.w = (int)mx8_encode4((uint32_t)e.z, (uint32_t)e.w, byte1);
  }
  uint8_t* dst = blob + kHeaderBytes + (size_t)frag * 2048 + 32 * L;
  *reinterpret_cast<v4i*>(dst) = lo;
  *reinterpret_cast<v4i*>(dst + 16) = hi;
  // scale record (s = c / 2, g), byte 2L + (c % 2): block 2c + L/32, i.e. this lane group's block
  uint8_t* sc = blob + blob_scales_offset(FMT_MX8, Np, K);
  sc[((size_t)(c / 2) * (Np / 32) + g) * 128 + 2 * L + (c & 1)] = (uint8_t)(h ? byte1 : byte0);
}

// NVFP4: the header (and a cleared tensor-maximum slot) first, in a launch of its own,
// so that the tensor maximum can be merged into the slot before the codes are packed.
__global__ void nv4_header_kernel(uint8_t* blob, int epi, int N, int K, int Np) {
  write_header(blob, FMT_NV4, epi, N, K, Np);       // zeroes the slot and the tensor scale
}

// NVFP4 codes: one thread per (fragment, lane) as FP4; the lane's 32 elements are two
// 16-element blocks (4c + 2h and 4c + 2h + 1 of the row, h = L/32), each with its own
// E4M3 scale.  Scale record (s = c/2, g): 256 bytes, byte 4L + 2(c%2) + b.
__global__ __launch_bounds__(256) void pack_nv4_kernel(const uint16_t* __restrict__ w, int N, int K,
                                                       int ldw, int epi, int Np,
                                                       uint8_t* __restrict__ blob) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  const uint32_t kc = (uint32_t)K / 64;
  const uint32_t total = (uint32_t)Np / 32 * kc * 64;
  const float st = nv4_tensor_scale(*reinterpret_cast<const uint32_t*>(blob + kNvAmaxOff));
  const float six_st = 6.0f * st;
  if (t == 0) *reinterpret_cast<float*>(blob + kNvTensorScaleOff) = st;
  if (t >= total) return;
  const uint32_t L = t & 63, frag = t >> 6;
  const uint32_t c = frag % kc, g = frag / kc;
  const int p = (int)(32 * g + (L & 31));
  const int src = packed_row_source(epi, N, p);
  v4i out = {0, 0, 0, 0};
  uint32_t sb0 = 0, sb1 = 0;
  if (src >= 0) {
    const v4i* wp = reinterpret_cast<const v4i*>(w + (size_t)src * ldw + 64 * c + 32 * (L >> 5));
    const v4i v0 = wp[0], v1 = wp[1], v2 = wp[2], v3 = wp[3];
    sb0 = nv4_scale_code(__uint_as_float(max(absmax8(v0), absmax8(v1)) << 16) / six_st);
    sb1 = nv4_scale_code(__uint_as_float(max(absmax8(v2), absmax8(v3)) << 16) / six_st);
    const float d0 = __builtin_amdgcn_cvt_f32_fp8((int)sb0, 0) * st;
    const float d1 = __builtin_amdgcn_cvt_f32_fp8((int)sb1, 0) * st;
    out.x = (int)nv4_encode8(v0, d0);
    out.y = (int)nv4_encode8(v1, d0);
    out.z = (int)nv4_encode8(v2, d1);
    out.w = (int)nv4_encode8(v3, d1);
  }
  *reinterpret_cast<v4i*>(blob + kHeaderBytes + (size_t)frag * 1024 + 16 * L) = out;
  uint8_t* sc = blob + blob_scales_offset(FMT_NV4, Np, K) + ((size_t)(c / 2) * (Np / 32) + g) * 256 + 4 * L +
                2 * (c & 1);
  sc[0] = (uint8_t)sb0;
  sc[1] = (uint8_t)sb1;
}

// FP8: one wave per packed row.  Pass 1 finds the row's amax (-> s_w), pass 2
// encodes 16-element runs; run r (k = 16r ..) lands in fragment (g, r/4), lane
// p%32 + 32*(r%2), byte 16*((r/2)%2) (the 8-bit fragment order above).
__global__ __launch_bounds__(256) void pack_fp8_kernel(const uint16_t* __restrict__ w, int N, int K,
                                                       int ldw, int epi, int Np,
                                                       uint8_t* __restrict__ blob) {
  const int lane = threadIdx.x & 63;
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blockIdx.x == 0 && threadIdx.x == 0) write_header(blob, FMT_FP8, epi, N, K, Np);
  if (p >= Np) return;
  const int src = packed_row_source(epi, N, p);
  float* sw = reinterpret_cast<float*>(blob + blob_scales_offset(FMT_FP8, Np, K));
  const int g = p / 32, kc = K / 64;
  const int lane_in_frag = p & 31;
  auto run_dst = [&](int r) {
    return blob + kHeaderBytes + ((size_t)g * kc + r / 4) * 2048 + 32 * (lane_in_frag + 32 * (r & 1)) +
           16 * ((r >> 1) & 1);
  };
  if (src < 0) {
    for (int r = lane; r < K / 16; r += 64) *reinterpret_cast<v4i*>(run_dst(r)) = v4i{0, 0, 0, 0};
    if (lane == 0) sw[p] = 0.0f;
    return;
  }
  const uint16_t* wr = w + (size_t)src * ldw;
  uint32_t m = 0;
  for (int k = lane * 8; k < K; k += 512) m = max(m, absmax8(*reinterpret_cast<const v4i*>(wr + k)));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  const float s = fp8_row_scale(m);
  if (lane == 0) sw[p] = s;
  for (int r = lane; r < K / 16; r += 64) {
    const v4i* wp = reinterpret_cast<const v4i*>(wr + 16 * r);
    const v4i a = wp[0], b = wp[1];
    v4i q;
    q.x = (int)fp8_encode4((uint32_t)a.x, (uint32_t)a.y, s);
    q.y = (int)fp8_encode4((uint32_t)a.z, (uint32_t)a.w, s);
    q.z = (int)fp8_encode4((uint32_t)b.x, (uint32_t)b.y, s);
    q.w = (int)fp8_encode4((uint32_t)b.z, (uint32_t)b.w, s);
    *reinterpret_cast<v4i*>(run_dst(r)) = q;
  }
}

}  // namespace

hipError_t launch_pack(int fmt, int epi, const uint16_t* w, int N, int K, int ldw, uint8_t* blob,
                       hipStream_t stream) {
  const int Np = padded_rows(N);
  if (fmt == FMT_NV4) {
    // header + cleared slot, the tensor maximum of W (logical rows; padding rows are
    // zero), then the codes and scales.  The tensor maximum's per-workgroup maxima go
    // to the start of the code area (at least 8 KB), which the packer then overwrites.
    hipLaunchKernelGGL(nv4_header_kernel, dim3(1), dim3(1), 0, stream, blob, epi, N, K, Np);
    static_assert(kNvPartialBytes <= 64 * 256 / 2, "the smallest code area holds the work space");
    if (hipError_t e = launch_amax_bf16(w, N, K, ldw, reinterpret_cast<uint32_t*>(blob + kNvAmaxOff),
                                        reinterpret_cast<uint32_t*>(blob + kHeaderBytes), stream))
      return e;
    const uint32_t total = (uint32_t)Np / 32 * ((uint32_t)K / 64) * 64;
    hipLaunchKernelGGL(pack_nv4_kernel, dim3((total + 255) / 256), dim3(256), 0, stream, w, N, K, ldw, epi, Np,
                       blob);
  } else if (fmt == FMT_FP4 || fmt == FMT_MX8) {
    const uint32_t total = (uint32_t)Np / 32 * ((uint32_t)K / 64) * 64;
    hipLaunchKernelGGL(fmt == FMT_FP4 ? pack_fp4_kernel : pack_mx8_kernel, dim3((total + 255) / 256), dim3(256), 0,
                       stream, w, N, K, ldw, epi, Np, blob);
  } else {
    hipLaunchKernelGGL(pack_fp8_kernel, dim3((Np + 3) / 4), dim3(256), 0, stream, w, N, K, ldw, epi, Np,
                       blob);
  }
  return hipGetLastError();
}

}  // namespace ditq
