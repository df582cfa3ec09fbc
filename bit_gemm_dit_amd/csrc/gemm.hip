// Fused low-bit GEMM + epilogue on gfx950 scaled MFMA.
//
// out = epi(A W^T): A = on-the-fly quantized activations [M, K] (row-major codes),
// W = packed weights (fragment layout, include/ditq.h).  The small op after the
// GEMM runs on the fp32 accumulators in registers and the result is written to
// HBM once as bf16 ("epilogue fusion": page "How fal made Ideogram V4 6x faster",
// paragraph 3; gated-SiLU with interleaved columns: paragraph 4; FP8 as the second
// precision: page "WaveSpeedAI X DataCrunch", engine list).
//
// Mapping to CDNA4:
// * MFMA operand A = a 32-row weight fragment, operand B = 32 tokens, so the
//   32x32 result tile of a lane is one token (lane % 32) by 16 output features
//   (n = 8*(r/4) + 4*(lane/32) + r%4 for accumulator register r).  A per-token
//   reduction over a head is then lane-local plus one exchange with lane ^ 32,
//   and a gate row and its up row (interleaved by the packer) meet in the same
//   lane and register of two adjacent tiles.
// * FP4: v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands (4 VGPRs) and the
//   E8M0 block scales applied by the instruction (op_sel picks the byte of the
//   64-K step).  FP8: the same instruction with E4M3 operands (8 VGPRs) and unit
//   block scales; the fp32 row/column scales are applied in the epilogue.
// * A workgroup computes a 256 (features) x 256 (tokens) tile with 8 waves (two per
//   SIMD, 128 accumulators each).  The large tile keeps the L2 -> LDS traffic at
//   about half of what the CU's load path can move while the MFMAs run at full
//   rate; two waves per SIMD let one wave's LDS waits overlap the other's MFMAs.
// * K advances in steps of 64 operand bytes per row (FP4: 128 K, FP8: 64 K)
//   through a 4-stage LDS ring filled by direct-to-LDS buffer loads, three steps
//   ahead of the MFMAs; one barrier per step.  Each stage also carries the step's
//   E8M0 scale bytes.  Weight tiles are copied verbatim (the blob is in lane
//   order); activation rows get a 16-byte XOR swizzle so fragment reads are free
//   of LDS bank conflicts.
// * Raw buffer loads return zeros past the end of a tensor, which clips ragged M
//   without branches; stores are predicated per row.
// * Workgroups are re-ordered so each XCD (workgroup id mod 8) walks a compact
//   band of output tiles and shares operand rows through its own L2.
#include "common.hpp"

namespace ditq {
namespace {

constexpr int kRowBytes = 64;    // operand bytes per row per k-step
constexpr int kStages = 4;       // LDS ring depth
constexpr int kGroupM = 4;       // tile-order group height (in M tiles)

template <int FMT_, int EPI_, int WN_, int WM_, int WAVES_N_, int WAVES_M_>
struct Tile {
  static constexpr int FMT = FMT_, EPI = EPI_;
  static constexpr int WN = WN_, WM = WM_, WAVES_N = WAVES_N_, WAVES_M = WAVES_M_;
  static constexpr int TN = WN / 32, TM = WM / 32;
  static constexpr int BN = WN * WAVES_N, BM = WM * WAVES_M;
  static constexpr int NW = WAVES_N * WAVES_M;
  static constexpr int NT = 64 * NW;
  static constexpr int CH = FMT == FMT_FP4 ? 2 : 1;         // 64-K MFMA steps per k-step
  static constexpr int KSTEP = 64 * CH;
  static constexpr int FRAG = FMT == FMT_FP4 ? 1024 : 2048;  // bytes of one 32x64 operand fragment
  static constexpr int GROUP_BYTES = FRAG * CH;              // one 32-row group per k-step (2 KB)
  // LDS stage: weight codes | activation codes | weight scale records | activation scales
  static constexpr int W_BYTES = BN * kRowBytes, A_BYTES = BM * kRowBytes;
  static constexpr int WS_OFF = W_BYTES + A_BYTES;
  static constexpr int WS_BYTES = FMT == FMT_FP4 ? BN / 32 * 128 : 0;   // 128 B per 32-row group
  static constexpr int AS_OFF = WS_OFF + WS_BYTES;
  static constexpr int AS_BYTES = FMT == FMT_FP4 ? BM * 4 : 0;          // 4 B per token
  static constexpr int STAGE = AS_OFF + AS_BYTES;
  // direct-to-LDS copies per wave per stage (plus one scale copy on waves 0 and 1 for FP4)
  static constexpr int WCK = W_BYTES / 1024 / NW;
  static constexpr int ACK = A_BYTES / 1024 / NW;
  static constexpr int VMEM_PER_STAGE = WCK + ACK;   // the fewest any wave issues per stage
  static_assert(W_BYTES % (1024 * NW) == 0 && A_BYTES % (1024 * NW) == 0, "whole 1 KB copies per wave");
  static_assert(WS_BYTES <= 1024 && AS_BYTES <= 1024, "each scale record set is one copy");
  static_assert(GROUP_BYTES == 2048, "a 32-row group moves 2 KB per k-step");
  static_assert(kStages * STAGE <= 160 * 1024, "the LDS ring must fit in a CU's LDS");
  static_assert(NW % 4 == 0, "whole waves per SIMD");
};

struct Params {
  const uint8_t* a_codes;
  const void* a_scales;       // FP4: u8 [M][K/32]; FP8: f32 [M]
  const uint8_t* w_codes;     // blob + header
  const void* w_scales;       // FP4: E8M0 groups; FP8: f32 [Np]
  uint16_t* out;
  int M, N, K, ldo;
  int tiles_m, tiles_n;
  uint32_t a_bytes, w_bytes, as_bytes, ws_bytes;
  const float* gamma_q;
  const float* gamma_k;
  float eps;
  int n_heads;
};

// Activation LDS rows are 64 bytes = 4 chunks of 16 bytes; chunk c of row r is
// stored at slot c ^ swz(r).  For a fixed logical chunk, rows r..r+7 (one 32-bank
// cycle of 16-byte reads) and r..r+15 (one 64-bank cycle) land in distinct banks.
__device__ __host__ constexpr int swz(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

__device__ inline void tile_coords(int bid, int total, int tiles_m, int tiles_n, int& tm, int& tn) {
  // workgroup ids are dealt round-robin to the 8 XCDs; give XCD x a contiguous range
  const int q = total >> 3, r = total & 7;
  const int x = bid & 7, i = bid >> 3;
  const int t = x * q + min(x, r) + i;
  // grouped order inside the range: kGroupM tiles down M, then across N
  const int per_group = kGroupM * tiles_n;
  const int group = t / per_group;
  const int first = group * kGroupM;
  const int gsz = min(tiles_m - first, kGroupM);
  const int w = t - group * per_group;
  tm = first + w % gsz;
  tn = w / gsz;
}

__device__ inline uint32_t pack_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, bf16x2));
}

// Store one 32x32 result tile of this lane (16 values, see the layout above) as
// bf16.  Partner lanes (lane, lane ^ 32) swap half-groups first so that each lane
// owns two runs of 8 consecutive columns: [8h, 8h+8) and [16+8h, 16+8h+8).
__device__ inline void store_tile(uint16_t* __restrict__ out, int ldo, int row, bool row_ok, int col0,
                                  int ncols, int h, const float* v) {
  uint32_t g[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    g[2 * i] = pack_bf16(v[4 * i], v[4 * i + 1]);
    g[2 * i + 1] = pack_bf16(v[4 * i + 2], v[4 * i + 3]);
  }
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    // permlane32_swap(a, b): lanes 32..63 of a <-> lanes 0..31 of b
    auto s = __builtin_amdgcn_permlane32_swap(g[0 + d], g[2 + d], false, false);
    g[0 + d] = s[0];
    g[2 + d] = s[1];
    auto t = __builtin_amdgcn_permlane32_swap(g[4 + d], g[6 + d], false, false);
    g[4 + d] = t[0];
    g[6 + d] = t[1];
  }
  if (row_ok) {
    uint16_t* o = out + (size_t)row * ldo;
    const int c0 = col0 + 8 * h, c1 = col0 + 16 + 8 * h;
    if (c0 < ncols) *reinterpret_cast<v4i*>(o + c0) = v4i{(int)g[0], (int)g[1], (int)g[2], (int)g[3]};
    if (c1 < ncols) *reinterpret_cast<v4i*>(o + c1) = v4i{(int)g[4], (int)g[5], (int)g[6], (int)g[7]};
  }
}

// SiLU(x) = x / (1 + e^-x) with the hardware exp2 and reciprocal (about 1 ulp
// each).  For very negative x, e^-x = inf and the result is -0, never NaN.
__device__ inline float silu(float x) {
  const float e = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}


// Operand fragments of one 64-K MFMA step: TN weight fragments, TM token fragments.
template <class T>
struct Frags {
  v8i w[T::TN];
  v8i a[T::TM];
};

template <class T, int J>
__device__ __forceinline__ void load_frags(Frags<T>& f, const uint8_t* stage, int wn, int wm, int lane) {
  const int h = lane >> 5, l32 = lane & 31;
  const uint8_t* wb = stage;
  const uint8_t* ab = stage + T::W_BYTES;
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn) {
    const uint8_t* fp = wb + (wn * T::TN + tn) * T::GROUP_BYTES + J * T::FRAG;
    if constexpr (T::FMT == FMT_FP4) {
      const v4i x = *reinterpret_cast<const v4i*>(fp + 16 * lane);
      f.w[tn] = __builtin_shufflevector(x, x, 0, 1, 2, 3, -1, -1, -1, -1);
    } else {
      const v4i x0 = *reinterpret_cast<const v4i*>(fp + 32 * lane);
      const v4i x1 = *reinterpret_cast<const v4i*>(fp + 32 * lane + 16);
      f.w[tn] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm) {
    const int r = wm * T::WM + 32 * tm + l32;
    const uint8_t* row = ab + r * kRowBytes;
    if constexpr (T::FMT == FMT_FP4) {
      const int c = 2 * J + h;
      const v4i x = *reinterpret_cast<const v4i*>(row + 16 * (c ^ swz(r)));
      f.a[tm] = __builtin_shufflevector(x, x, 0, 1, 2, 3, -1, -1, -1, -1);
    } else {
      const int c = 2 * h;
      const v4i x0 = *reinterpret_cast<const v4i*>(row + 16 * (c ^ swz(r)));
      const v4i x1 = *reinterpret_cast<const v4i*>(row + 16 * ((c + 1) ^ swz(r)));
      f.a[tm] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

// sched_group_barrier masks
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Scale words of one k-step (FP4): the weight record's 16-bit word per lane holds
// op_sel bytes 0 and 1; a token's 4 scale bytes are its blocks 0..3 of the step,
// and this lane's MFMA steps j = 0, 1 take blocks 2j + h (selector byte 0x0C
// gives a zero byte).
template <class T>
struct Scales {
  uint32_t w[T::TN];
  uint32_t a[T::TM];
};

// Raw scale words of a stage (the activation bytes are selected later, once the
// LDS reads have landed, so that no MFMA waits on them).
template <class T>
__device__ __forceinline__ void load_scales(Scales<T>& sc, const uint8_t* stage, int wn, int wm, int lane) {
  if constexpr (T::FMT == FMT_FP4) {
    const int l32 = lane & 31;
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn)
      sc.w[tn] = *reinterpret_cast<const uint16_t*>(stage + T::WS_OFF + (wn * T::TN + tn) * 128 + 2 * lane);
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm)
      sc.a[tm] = *reinterpret_cast<const uint32_t*>(stage + T::AS_OFF + 4 * (wm * T::WM + 32 * tm + l32));
  } else {
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn) sc.w[tn] = 0;
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) sc.a[tm] = 0;
  }
}

template <class T>
__device__ __forceinline__ void select_scales(Scales<T>& sc, int lane) {
  if constexpr (T::FMT == FMT_FP4) {
    const uint32_t sel = (lane & 32) ? 0x0C0C0301u : 0x0C0C0200u;
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) sc.a[tm] = __builtin_amdgcn_perm(0u, sc.a[tm], sel);
  }
}

// MFMAs of 64-K step J over token tiles [TM0, TM1), with the LDS reads that are
// issued in the same region spread between them.
template <class T, int J, int TM0, int TM1>
__device__ __forceinline__ void mfma_part(v16f (&acc)[T::TN][T::TM], const Frags<T>& f, const Scales<T>& sc) {
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
    for (int tm = TM0; tm < TM1; ++tm) {
      if constexpr (T::FMT == FMT_FP4)
        acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[tn], f.a[tm], acc[tn][tm], 4, 4, J,
                                                                      (int)sc.w[tn], J, (int)sc.a[tm]);
      else
        acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[tn], f.a[tm], acc[tn][tm], 0, 0, 0,
                                                                      0x7F7F7F7F, 0, 0x7F7F7F7F);
    }
}

// Spread NDS LDS reads between NMFMA MFMAs of the current scheduling region.
template <int NMFMA, int NDS>
__device__ __forceinline__ void interleave() {
  constexpr int pairs = NDS < NMFMA ? NDS : NMFMA;
#pragma unroll
  for (int i = 0; i < pairs; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  if constexpr (NMFMA > pairs) __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMFMA - pairs, 0);
  if constexpr (NDS > pairs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NDS - pairs, 0);
}

// ---------------------------------------------------------------- epilogues
template <class T>
__device__ __forceinline__ void epilogue(const Params& p, v16f (&acc)[T::TN][T::TM], int n0w, int m0w, int lane) {
  const int h = lane >> 5, l32 = lane & 31;
  if constexpr (T::EPI == EPI_IDENTITY || T::EPI == EPI_GATED_SILU) {
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
      const int row = m0w + 32 * tm + l32;
      const bool ok = row < p.M;
      float sa = 1.0f;
      if constexpr (T::FMT == FMT_FP8) sa = reinterpret_cast<const float*>(p.a_scales)[ok ? row : p.M - 1];
      if constexpr (T::EPI == EPI_IDENTITY) {
#pragma unroll
        for (int tn = 0; tn < T::TN; ++tn) {
          float v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = acc[tn][tm][r];
          if constexpr (T::FMT == FMT_FP8) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const v4f sw = *reinterpret_cast<const v4f*>(
                  reinterpret_cast<const float*>(p.w_scales) + n0w + 32 * tn + 8 * g + 4 * h);
#pragma unroll
              for (int i = 0; i < 4; ++i) v[4 * g + i] *= sa * sw[i];
            }
          }
          store_tile(p.out, p.ldo, row, ok, n0w + 32 * tn, p.N, h, v);
        }
      } else {
#pragma unroll
        for (int q = 0; q < T::TN / 2; ++q) {
          float gate[16], up[16], v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            gate[r] = acc[2 * q][tm][r];
            up[r] = acc[2 * q + 1][tm][r];
          }
          if constexpr (T::FMT == FMT_FP8) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const float* ws = reinterpret_cast<const float*>(p.w_scales) + n0w + 64 * q + 8 * g + 4 * h;
              const v4f sg = *reinterpret_cast<const v4f*>(ws);
              const v4f su = *reinterpret_cast<const v4f*>(ws + 32);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                gate[4 * g + i] *= sa * sg[i];
                up[4 * g + i] *= sa * su[i];
              }
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = silu(gate[r]) * up[r];
          store_tile(p.out, p.ldo, row, ok, n0w / 2 + 32 * q, p.N / 2, h, v);
        }
      }
    }
  } else {
    // Per-head QK-RMSNorm; the wave's WN columns are exactly one head.
    constexpr int D = T::WN;
    const int head = n0w / D;
    const int part = head / p.n_heads;          // 0 = Q, 1 = K, 2 = V, 3 = padding past N
    if (part >= 3) return;
    const float* gamma = part == 0 ? p.gamma_q : p.gamma_k;
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
      const int row = m0w + 32 * tm + l32;
      const bool ok = row < p.M;
      if (part == 2) {
#pragma unroll
        for (int tn = 0; tn < T::TN; ++tn) {
          float v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = acc[tn][tm][r];
          store_tile(p.out, p.ldo, row, ok, n0w + 32 * tn, p.N, h, v);
        }
        continue;
      }
      // Revisit schedule: the first half of the head (tiles [0, TN/2)) keeps its
      // fp32 values and its partial sum of squares in registers while the second
      // half's partial sum is formed; the combined sum then normalises the second
      // half, which is stored, and the first half is revisited and stored.  For
      // head_dim 128 the same code runs over two 64-column halves.
      float ss_first = 0.0f, ss_second = 0.0f;
#pragma unroll
      for (int tn = 0; tn < T::TN / 2; ++tn)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss_first += acc[tn][tm][r] * acc[tn][tm][r];
#pragma unroll
      for (int tn = T::TN / 2; tn < T::TN; ++tn)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss_second += acc[tn][tm][r] * acc[tn][tm][r];
      float ss = ss_first + ss_second;
      ss += __shfl_xor(ss, 32);                   // the partner lane holds the other 16 rows of each tile
      const float rs = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps);
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        const int t0 = step == 0 ? T::TN / 2 : 0;   // second half first, then revisit the first
#pragma unroll
        for (int tn = t0; tn < t0 + T::TN / 2; ++tn) {
          float v[16];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const v4f gm = *reinterpret_cast<const v4f*>(gamma + 32 * tn + 8 * g + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) v[4 * g + i] = acc[tn][tm][4 * g + i] * rs * gm[i];
          }
          store_tile(p.out, p.ldo, row, ok, n0w + 32 * tn, p.N, h, v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- kernel
// An empty volatile asm that reads every accumulator: the MFMAs of a k-step must
// then be issued before it, and it stays ordered with the wait and the barrier that
// follow (MFMAs touch no memory, so without it they may be sunk below the barrier).
// The asm exists only in the device pass: on the host pass "a" would name an x86
// register, and the failed constraint would silently drop the kernel's host stub.
template <class T>
__device__ __forceinline__ void pin_accumulators(v16f (&acc)[T::TN][T::TM]) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) asm volatile("" ::"a"(acc[tn][tm]));
#endif
}

// N direct-to-LDS copies of BYTES per lane each: lane L of copy i fetches BYTES at
// voff[i] + soff and the hardware writes them to dst + 64*BYTES*i + BYTES*L.
// (A plain device function: inside a lambda the builtin would also be compiled
// for the host, where it fails and takes the kernel's host stub with it.)
template <int N, int BYTES>
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, const uint32_t* voff, int soff,
                                            uint8_t* dst) {
  static_assert(BYTES == 16 || BYTES == 4, "copy width");
#pragma unroll
  for (int i = 0; i < N; ++i) {
    auto* d = (__attribute__((address_space(3))) void*)(dst + 64 * BYTES * i);
    if constexpr (BYTES == 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, d, 16, voff[i], soff, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, d, 4, voff[i], soff, 0, 0);
  }
}

// s_waitcnt vmcnt(n) with the other counters unconstrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <class T>
__global__ void __launch_bounds__(T::NT, T::NW / 4) gemm_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * T::STAGE];
  // readfirstlane: the wave index is uniform, and the compiler must know it (a
  // per-wave buffer descriptor would otherwise become a loop over lanes)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % T::WAVES_N, wm = wave / T::WAVES_N;
  int tmi, tni;
  tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tmi, tni);
  const int n0 = tni * T::BN, m0 = tmi * T::BM;
  const int nks = p.K / T::KSTEP;
  const uint32_t wgroup = (uint32_t)(p.K / 64) * T::FRAG;

  const auto a_rsrc = make_rsrc(p.a_codes, p.a_bytes);
  const auto w_rsrc = make_rsrc(p.w_codes, p.w_bytes);

  // Direct-to-LDS copies (each wave instruction writes 64 lanes x 16 bytes = 1 KB):
  // weight copy q = half of row group q/2 (verbatim: the blob is in lane order);
  // activation copy q = 16 token rows of the K panel (contiguous 1 KB in the
  // panel-major layout), lane L fetching the logical chunk that the swizzle
  // places at slot L%4 of row 16q + L/4.
  uint32_t w_off[T::WCK], a_off[T::ACK];
#pragma unroll
  for (int i = 0; i < T::WCK; ++i) {
    const int q = wave * T::WCK + i;
    w_off[i] = (uint32_t)(n0 / 32 + (q >> 1)) * wgroup + 1024u * (q & 1) + 16u * lane;
  }
#pragma unroll
  for (int i = 0; i < T::ACK; ++i) {
    const int q = wave * T::ACK + i;
    const int r = 16 * q + (lane >> 2);
    const int c = (lane & 3) ^ swz(r);
    // Rows past M read the next panel's codes (or zeros past the buffer end);
    // their results are never stored.
    a_off[i] = (uint32_t)(m0 + r) * kRowBytes + 16u * c;
  }
  const uint32_t a_panel = (uint32_t)p.M * kRowBytes;   // bytes of one K panel of the activation codes
  // FP4 scale copies, one per stage: wave 0 copies the weight scale records of the
  // block's row groups (1 KB, contiguous for one K step), wave 1 the 4-byte scale
  // words of the block's tokens (BM * 4 bytes, contiguous in the panel-major layout).
  [[maybe_unused]] __amdgpu_buffer_rsrc_t s_rsrc;
  uint32_t s_off[1] = {0};
  [[maybe_unused]] uint32_t s_step = 0;
  [[maybe_unused]] bool s_active = false;
  [[maybe_unused]] int s_dst = 0;
  if constexpr (T::FMT == FMT_FP4) {
    if (wave == 0) {
      s_rsrc = make_rsrc(p.w_scales, p.ws_bytes);
      s_off[0] = (uint32_t)(n0 / 32) * 128u + 16u * lane;
      s_step = (uint32_t)(padded_rows(p.N) / 32) * 128u;
      s_dst = T::WS_OFF;
      s_active = 16 * lane < T::WS_BYTES;
    } else if (wave == 1) {
      s_rsrc = make_rsrc(p.a_scales, p.as_bytes);
      s_off[0] = (uint32_t)m0 * 4u + 16u * lane;
      s_step = (uint32_t)p.M * 4u;
      s_dst = T::AS_OFF;
      s_active = 16 * lane < T::AS_BYTES;
    }
  }

  auto issue_stage = [&](int ks) {
    uint8_t* base = lds + (ks % kStages) * T::STAGE;
    copy_to_lds<T::WCK, 16>(w_rsrc, w_off, ks * T::GROUP_BYTES, base + wave * T::WCK * 1024);
    copy_to_lds<T::ACK, 16>(a_rsrc, a_off, ks * a_panel, base + T::W_BYTES + wave * T::ACK * 1024);
    if constexpr (T::FMT == FMT_FP4) {
      if (s_active) copy_to_lds<1, 16>(s_rsrc, s_off, ks * s_step, base + s_dst);
    }
  };

  v16f acc[T::TN][T::TM];
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) acc[tn][tm] = v16f{};

  // Pipeline.  Step ks computes from ring slot ks % kStages.  The barrier of step ks
  // sits between its two halves of MFMAs: before it the wave has issued the first
  // half (which keeps the MFMA pipe busy through the wait), after it stage ks+1 is
  // visible to every wave and slot ks % kStages is free, so the copy of stage
  // ks + kStages goes there and the next stage's first fragments are read while
  // the second half of the MFMAs runs.  Copies are issued for every step up to
  // nks + kStages - 1: those past the end of K read zeros or unused rows (the
  // buffer descriptors bound every read) into slots that are no longer read,
  // which keeps the wait counts constant and the loop body free of branches.
  auto stage_ptr = [&](int ks) { return lds + (ks % kStages) * T::STAGE; };

#pragma unroll
  for (int i = 0; i < kStages; ++i) issue_stage(i);
  wait_vmcnt<(kStages - 1) * T::VMEM_PER_STAGE>();   // stage 0 has landed
  __syncthreads();
  Frags<T> fa, fb;
  Scales<T> sc, sn;
  load_scales<T>(sc, stage_ptr(0), wn, wm, lane);
  load_frags<T, 0>(fa, stage_ptr(0), wn, wm, lane);
  select_scales<T>(sc, lane);
  constexpr int NDS = (T::TN + T::TM) * (T::FMT == FMT_FP4 ? 1 : 2);
  constexpr int NSC = T::FMT == FMT_FP4 ? T::TN + T::TM : 0;
  for (int ks = 0; ks < nks; ++ks) {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (T::CH == 2) {
      // first half: MFMA step 0 of stage ks, reading step 1's fragments meanwhile
      load_frags<T, 1>(fb, stage_ptr(ks), wn, wm, lane);
      mfma_part<T, 0, 0, T::TM>(acc, fa, sc);
      interleave<T::TN * T::TM, NDS>();
    } else {
      mfma_part<T, 0, 0, T::TM / 2>(acc, fa, sc);
    }
    pin_accumulators<T>(acc);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(kStages - 2) * T::VMEM_PER_STAGE>();   // stage ks+1 has landed
    __syncthreads();
    issue_stage(ks + kStages);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (T::CH == 2) {
      // second half: MFMA step 1 of stage ks, reading stage ks+1's step-0 operands
      load_scales<T>(sn, stage_ptr(ks + 1), wn, wm, lane);
      load_frags<T, 0>(fa, stage_ptr(ks + 1), wn, wm, lane);
      mfma_part<T, 1, 0, T::TM>(acc, fb, sc);
      interleave<T::TN * T::TM, NDS + NSC>();
      pin_accumulators<T>(acc);
      __builtin_amdgcn_sched_barrier(0);
      sc = sn;
      select_scales<T>(sc, lane);
    } else {
      load_frags<T, 0>(fb, stage_ptr(ks + 1), wn, wm, lane);
      mfma_part<T, 0, T::TM / 2, T::TM>(acc, fa, sc);
      interleave<T::TN * (T::TM - T::TM / 2), NDS>();
      pin_accumulators<T>(acc);
      __builtin_amdgcn_sched_barrier(0);
      fa = fb;
    }
  }
  wait_vmcnt<0>();     // no copy into this workgroup's LDS may outlive it
  __builtin_amdgcn_sched_barrier(0);
  epilogue<T>(p, acc, n0 + wn * T::WN, m0 + wm * T::WM, lane);
}

template <class T>
hipError_t launch(Params& p, hipStream_t stream) {
  p.tiles_m = (p.M + T::BM - 1) / T::BM;
  p.tiles_n = padded_rows(p.N) / T::BN;
  const int grid = p.tiles_m * p.tiles_n;
  hipLaunchKernelGGL(gemm_kernel<T>, dim3(grid), dim3(T::NT), 0, stream, p);
  return hipGetLastError();
}

Params make_params(const uint8_t* a_codes, const void* a_scales, const uint8_t* blob, int fmt, int M, int N,
                   int K, uint16_t* out, int ldo) {
  const int Np = padded_rows(N);
  Params p{};
  p.a_codes = a_codes;
  p.a_scales = a_scales;
  p.w_codes = blob + kHeaderBytes;
  p.w_scales = blob + blob_scales_offset(fmt, Np, K);
  p.out = out;
  p.M = M;
  p.N = N;
  p.K = K;
  p.ldo = ldo;
  p.a_bytes = (uint32_t)((size_t)M * (fmt == FMT_FP4 ? K / 2 : K));
  p.w_bytes = (uint32_t)blob_code_bytes(fmt, Np, K);
  p.as_bytes = (uint32_t)((size_t)M * (fmt == FMT_FP4 ? K / 32 : 4));
  p.ws_bytes = (uint32_t)blob_scale_bytes(fmt, Np, K);
  return p;
}

}  // namespace

hipError_t launch_gemm_fp4(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* blob, int M, int N,
                           int K, int epi, const RmsArgs* rms, uint16_t* out, int ldo, hipStream_t stream) {
  Params p = make_params(a_codes, a_scales, blob, FMT_FP4, M, N, K, out, ldo);
  switch (epi) {
    case EPI_IDENTITY:
      return launch<Tile<FMT_FP4, EPI_IDENTITY, 128, 64, 2, 4>>(p, stream);
    case EPI_GATED_SILU:
      return launch<Tile<FMT_FP4, EPI_GATED_SILU, 128, 64, 2, 4>>(p, stream);
    default:
      p.gamma_q = rms->gamma_q;
      p.gamma_k = rms->gamma_k;
      p.eps = rms->eps;
      p.n_heads = rms->n_heads;
      if (rms->head_dim == 128) return launch<Tile<FMT_FP4, EPI_QK_RMSNORM, 128, 64, 2, 4>>(p, stream);
      return launch<Tile<FMT_FP4, EPI_QK_RMSNORM, 256, 32, 1, 8>>(p, stream);
  }
}

hipError_t launch_gemm_fp8(const uint8_t* a_codes, const float* a_scales, const uint8_t* blob, int M, int N,
                           int K, int epi, uint16_t* out, int ldo, hipStream_t stream) {
  Params p = make_params(a_codes, a_scales, blob, FMT_FP8, M, N, K, out, ldo);
  if (epi == EPI_GATED_SILU) return launch<Tile<FMT_FP8, EPI_GATED_SILU, 128, 64, 2, 4>>(p, stream);
  return launch<Tile<FMT_FP8, EPI_IDENTITY, 128, 64, 2, 4>>(p, stream);
}

}  // namespace ditq
