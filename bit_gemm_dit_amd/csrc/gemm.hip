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
//   E8M0 block scales applied by the instruction: the scale dword of a lane holds
//   the scales of its four 64-K steps, picked with op_sel.  FP8: the same
//   instruction with E4M3 operands (8 VGPRs) and unit block scales; the fp32
//   row/column scales are applied in the epilogue.
// * One k-step moves 128 bytes per operand row (FP4: 256 K, FP8: 128 K) through
//   LDS, double-buffered: global loads of step k+1 are issued before the MFMAs of
//   step k and written to the other buffer after them; one barrier per step.
//   Weight tiles are copied verbatim (already in lane order); activation rows are
//   stored with a 16-byte XOR swizzle so fragment reads are bank-conflict free.
// * Raw buffer loads return zeros past the end of a tensor, which clips ragged M
//   without branches; stores are predicated per row.
// * Workgroups are re-ordered so each XCD (workgroup id mod 8) walks a compact
//   band of output tiles and shares operand rows through its own L2.
#include "common.hpp"

namespace ditq {
namespace {

constexpr int kRowBytes = 128;   // operand bytes per row per k-step
constexpr int kGroupM = 4;       // tile-order group height (in M tiles)

template <int FMT_, int EPI_, int WN_, int WM_, int WAVES_N_, int WAVES_M_>
struct Tile {
  static constexpr int FMT = FMT_, EPI = EPI_;
  static constexpr int WN = WN_, WM = WM_, WAVES_N = WAVES_N_, WAVES_M = WAVES_M_;
  static constexpr int TN = WN / 32, TM = WM / 32;
  static constexpr int BN = WN * WAVES_N, BM = WM * WAVES_M;
  static constexpr int NT = 64 * WAVES_N * WAVES_M;
  static constexpr int CH = FMT == FMT_FP4 ? 4 : 2;        // 64-K MFMA steps per k-step
  static constexpr int KSTEP = 64 * CH;
  static constexpr int FRAG = FMT == FMT_FP4 ? 1024 : 2048; // bytes of one 32x64 operand fragment
  static constexpr int W_BYTES = BN * kRowBytes, A_BYTES = BM * kRowBytes;
  static constexpr int STAGE = W_BYTES + A_BYTES;
  static constexpr int WCH = W_BYTES / 16 / NT, ACH = A_BYTES / 16 / NT;
  static_assert(W_BYTES % (16 * NT) == 0 && A_BYTES % (16 * NT) == 0, "tile copy must divide evenly");
  static_assert(FRAG * CH == 4096, "a 32-row group moves 4 KB per k-step");
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

// Activation LDS rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row r is
// stored at slot c ^ swz(r).  Eight consecutive rows (one 32-bank cycle of a
// 16-byte read) and sixteen consecutive rows (one 64-bank cycle) both map a fixed
// logical chunk to distinct banks.
__device__ __host__ constexpr int swz(int r) { return (r ^ (r >> 3)) & 7; }

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
__device__ __forceinline__ void load_frags(Frags<T>& f, const uint8_t* wb, const uint8_t* ab, int wn, int wm,
                                           int lane) {
  const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn) {
    const uint8_t* fp = wb + ((wn * T::TN + tn) * T::CH + J) * T::FRAG;
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
      const int c = 4 * J + 2 * h;
      const v4i x0 = *reinterpret_cast<const v4i*>(row + 16 * (c ^ swz(r)));
      const v4i x1 = *reinterpret_cast<const v4i*>(row + 16 * ((c + 1) ^ swz(r)));
      f.a[tm] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

template <class T, int J>
__device__ __forceinline__ void mfma_frags(v16f (&acc)[T::TN][T::TM], const Frags<T>& f, const uint32_t* wsc,
                                           const uint32_t* asc) {
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
      if constexpr (T::FMT == FMT_FP4)
        acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[tn], f.a[tm], acc[tn][tm], 4, 4, J,
                                                                      (int)wsc[tn], J, (int)asc[tm]);
      else
        acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[tn], f.a[tm], acc[tn][tm], 0, 0, 0,
                                                                      0x7F7F7F7F, 0, 0x7F7F7F7F);
    }
}

// sched_group_barrier masks
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Issue order for one 64-K step: the LDS reads of the next step's fragments are
// spread between this step's MFMAs, so their latency hides behind MFMA work.
template <class T>
__device__ __forceinline__ void interleave_hint(bool next_loads) {
  constexpr int NMFMA = T::TN * T::TM;
  constexpr int NDS = (T::TN + T::TM) * (T::FMT == FMT_FP4 ? 1 : 2);
  if (next_loads) {
#pragma unroll
    for (int i = 0; i < NDS; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    if constexpr (NMFMA > NDS) __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMFMA - NDS, 0);
  } else {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, NMFMA, 0);
  }
}

// One k-step: fragments of 64-K step j+1 are read from LDS while the MFMAs of step
// j run (two register sets, f0 / f1).
template <class T>
__device__ __forceinline__ void compute_stage(v16f (&acc)[T::TN][T::TM], const uint8_t* stage, int wn, int wm,
                                              int lane, const uint32_t* wsc, const uint32_t* asc) {
  const uint8_t* wb = stage;
  const uint8_t* ab = stage + T::W_BYTES;
  Frags<T> f0, f1;
  load_frags<T, 0>(f0, wb, ab, wn, wm, lane);
  __builtin_amdgcn_sched_barrier(0);
  load_frags<T, 1>(f1, wb, ab, wn, wm, lane);
  mfma_frags<T, 0>(acc, f0, wsc, asc);
  interleave_hint<T>(true);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (T::CH == 4) {
    load_frags<T, 2>(f0, wb, ab, wn, wm, lane);
    mfma_frags<T, 1>(acc, f1, wsc, asc);
    interleave_hint<T>(true);
    __builtin_amdgcn_sched_barrier(0);
    load_frags<T, 3>(f1, wb, ab, wn, wm, lane);
    mfma_frags<T, 2>(acc, f0, wsc, asc);
    interleave_hint<T>(true);
    __builtin_amdgcn_sched_barrier(0);
    mfma_frags<T, 3>(acc, f1, wsc, asc);
    interleave_hint<T>(false);
  } else {
    mfma_frags<T, 1>(acc, f1, wsc, asc);
    interleave_hint<T>(false);
  }
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

// N direct-to-LDS copies of 1 KB each: lane L of copy i fetches 16 bytes at
// voff[i] + soff and the hardware writes them to dst + 1024 i + 16 L.
// (A plain device function: inside a lambda the builtin would also be compiled
// for the host, where it fails and takes the kernel's host stub with it.)
template <int N>
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, const uint32_t* voff, int soff,
                                            uint8_t* dst) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16,
                                             voff[i], soff, 0, 0);
}

// waitcnt immediates (gfx9 encoding: vmcnt[3:0]|expcnt[6:4]|lgkmcnt[11:8]|vmcnt_hi[15:14])
constexpr int kWaitVm0 = 0x0F70;   // vmcnt(0), others unconstrained

template <class T>
__global__ void __launch_bounds__(T::NT) gemm_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * T::STAGE];
  constexpr int NW = T::NT / 64;
  constexpr int WCK = T::W_BYTES / 1024 / NW;    // 1 KB LDS chunks per wave per k-step
  constexpr int ACK = T::A_BYTES / 1024 / NW;
  static_assert(T::W_BYTES % (1024 * NW) == 0 && T::A_BYTES % (1024 * NW) == 0, "chunks per wave");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % T::WAVES_N, wm = wave / T::WAVES_N;
  const int l32 = lane & 31;
  int tmi, tni;
  tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tmi, tni);
  const int n0 = tni * T::BN, m0 = tmi * T::BM;
  const int nks = p.K / T::KSTEP;
  const uint32_t arow = T::FMT == FMT_FP4 ? (uint32_t)p.K / 2 : (uint32_t)p.K;
  const uint32_t wgroup = (uint32_t)(p.K / 64) * T::FRAG;

  const auto a_rsrc = make_rsrc(p.a_codes, p.a_bytes);
  const auto w_rsrc = make_rsrc(p.w_codes, p.w_bytes);

  // Direct-to-LDS copies: each wave instruction writes 1 KB of LDS, lane L at +16L.
  // Weight chunk q = 1 KB of row group q/4 (copied verbatim: the blob is in lane
  // order already).  Activation chunk q = 8 rows of 128 bytes; lane L fetches the
  // logical 16-byte chunk that the swizzle places at slot L%8 of row 8q + L/8.
  uint32_t w_off[WCK], a_off[ACK];
#pragma unroll
  for (int i = 0; i < WCK; ++i) {
    const int q = wave * WCK + i;
    w_off[i] = (uint32_t)(n0 / 32 + (q >> 2)) * wgroup + 1024u * (q & 3) + 16u * lane;
  }
#pragma unroll
  for (int i = 0; i < ACK; ++i) {
    const int q = wave * ACK + i;
    const int r = 8 * q + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    a_off[i] = (uint32_t)(m0 + r) * arow + 16u * c;     // rows >= M lie past the buffer and read as 0
  }

  // E8M0 scales (FP4): one dword per weight row tile, 8 bytes per token row.
  [[maybe_unused]] __amdgpu_buffer_rsrc_t ws_rsrc, as_rsrc;
  uint32_t ws_off[T::TN], as_off[T::TM];
  uint32_t wsc[T::TN], asc[T::TM], wsc_n[T::TN];
  uint32_t asr_lo[T::TM], asr_hi[T::TM];
  const uint32_t perm_sel = (lane & 32) ? 0x07050301u : 0x06040200u;   // blocks 2j + h, j = 0..3
  if constexpr (T::FMT == FMT_FP4) {
    ws_rsrc = make_rsrc(p.w_scales, p.ws_bytes);
    as_rsrc = make_rsrc(p.a_scales, p.as_bytes);
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn)
      ws_off[tn] = (uint32_t)(n0 / 32 + wn * T::TN + tn) * (uint32_t)(p.K / 256) * 256u + 4u * lane;
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm)
      as_off[tm] = (uint32_t)(m0 + wm * T::WM + 32 * tm + l32) * (uint32_t)(p.K / 32);
  }
  auto issue_loads = [&](int ks, int buf) {
    if constexpr (T::FMT == FMT_FP4) {
#pragma unroll
      for (int tn = 0; tn < T::TN; ++tn)
        wsc_n[tn] = __builtin_amdgcn_raw_buffer_load_b32(ws_rsrc, ws_off[tn], ks * 256, 0);
#pragma unroll
      for (int tm = 0; tm < T::TM; ++tm) {
        const auto d = __builtin_amdgcn_raw_buffer_load_b64(as_rsrc, as_off[tm], ks * 8, 0);
        asr_lo[tm] = d[0];
        asr_hi[tm] = d[1];
      }
    }
    copy_to_lds<WCK>(w_rsrc, w_off, ks * 4096, lds + buf * T::STAGE + wave * WCK * 1024);
    copy_to_lds<ACK>(a_rsrc, a_off, ks * kRowBytes, lds + buf * T::STAGE + T::W_BYTES + wave * ACK * 1024);
  };
  auto take_scales = [&]() {
    if constexpr (T::FMT == FMT_FP4) {
#pragma unroll
      for (int tn = 0; tn < T::TN; ++tn) wsc[tn] = wsc_n[tn];
#pragma unroll
      for (int tm = 0; tm < T::TM; ++tm) asc[tm] = __builtin_amdgcn_perm(asr_hi[tm], asr_lo[tm], perm_sel);
    }
  };

  v16f acc[T::TN][T::TM];
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) acc[tn][tm] = v16f{};

  issue_loads(0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  take_scales();
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < nks;
    // the other buffer was last read in step ks-1, which every wave finished before the barrier
    if (more) issue_loads(ks + 1, cur ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage<T>(acc, lds + cur * T::STAGE, wn, wm, lane, wsc, asc);
    pin_accumulators<T>(acc);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);       // this wave's copies into the other buffer have landed
    if (more) take_scales();
    __syncthreads();                            // ... and every other wave's; all reads of `cur` are done
  }
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
      return launch<Tile<FMT_FP4, EPI_IDENTITY, 128, 128, 2, 2>>(p, stream);
    case EPI_GATED_SILU:
      return launch<Tile<FMT_FP4, EPI_GATED_SILU, 128, 128, 2, 2>>(p, stream);
    default:
      p.gamma_q = rms->gamma_q;
      p.gamma_k = rms->gamma_k;
      p.eps = rms->eps;
      p.n_heads = rms->n_heads;
      if (rms->head_dim == 128) return launch<Tile<FMT_FP4, EPI_QK_RMSNORM, 128, 128, 2, 2>>(p, stream);
      return launch<Tile<FMT_FP4, EPI_QK_RMSNORM, 256, 64, 1, 4>>(p, stream);
  }
}

hipError_t launch_gemm_fp8(const uint8_t* a_codes, const float* a_scales, const uint8_t* blob, int M, int N,
                           int K, int epi, uint16_t* out, int ldo, hipStream_t stream) {
  Params p = make_params(a_codes, a_scales, blob, FMT_FP8, M, N, K, out, ldo);
  if (epi == EPI_GATED_SILU) return launch<Tile<FMT_FP8, EPI_GATED_SILU, 128, 128, 2, 2>>(p, stream);
  return launch<Tile<FMT_FP8, EPI_IDENTITY, 128, 128, 2, 2>>(p, stream);
}

}  // namespace ditq
