// Fused low-bit GEMM + epilogue on gfx950 scaled MFMA.
//
// out = epi(A W^T): A = on-the-fly quantized activations [M, K] (K-panel-major
// codes), W = packed weights (MFMA fragment layout, include/ditq.h).  The small op
// after the GEMM runs on the fp32 accumulators in registers and the result is
// written to HBM once as bf16 ("epilogue fusion": page "How fal made Ideogram V4 6x
// faster", paragraph 3; gated-SiLU with interleaved columns: paragraph 4; FP8 as the
// second precision: page "WaveSpeedAI X DataCrunch", engine list).  The other small
// ops of a DiT block fuse the same way: the MLP's GELU (tanh form; fused GELU:
// page on Google's on-device diffusion work, laaro.com) and the gated residual
// update out = residual + gate * C of adaLN-style blocks.
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
//   64-K step).  MXFP8: the same with E4M3 operands (8 VGPRs) and E8M0 block
//   scales, in the FP4 path's k-step of two 64-K units.  FP8: E4M3 operands and
//   unit block scales; the fp32 row/column scales are applied in the epilogue.
// * NVFP4 (E2M1 with E4M3 scales per 16 K and an fp32 tensor scale): the block-scaled
//   MFMA takes only power-of-two scales per 32 K, so the FP4 fragments are
//   dequantized in registers instead: E2M1 -> f16 (exact), times the E4M3 block
//   scale as a packed f16 multiply (exact: at most 6 significant bits, within f16's
//   range), into v_mfma_f32_32x32x16_f16 (four per 64-K unit); the two tensor scales
//   multiply the accumulator in the epilogue.  Same loads, stages and lane layouts as
//   FP4, at the f16 MFMA rate.
// * A workgroup of 4 waves (one per SIMD) computes a 256 (features) x BM (tokens)
//   tile, on one of two wave grids:
//   - 4 x 1 (FP8 with the identity, gated-SiLU and GELU epilogues; FP4 with those
//     where K / 128 is not a multiple of 6): wave wn owns 64 features x all BM
//     tokens (2 x 6 result tiles of 32 x 32, BM = 192).  No weight row is needed by
//     two waves, so every weight fragment is loaded straight into a ring of
//     registers several 64-K steps ahead, and only the activation tile is shared.
//   - 2 x 2 (the other formats and epilogues): wave (wn, wm) owns 128 features x
//     BM/2 tokens (4 x TM result tiles, TM = 3 or 4).  A head of QK-RMSNorm is then
//     one or two waves wide.  Of each wave's 4 weight row groups, FP4 and FP8
//     stage 2 through LDS (one copy per workgroup, read by the two waves of a row
//     band) and load 2 into the register ring; MXFP8 and NVFP4 load all 4 into
//     registers, and so do FP4 identity, gated-SiLU, GELU and the gated residual
//     where K / 128 is a multiple of 6, and FP4 QK-RMSNorm head_dim 128 in
//     192-token tiles (each wave then reads only its half of the tile's token rows
//     from LDS, at the price of the two waves of a row band both loading its
//     weights).
//   The blob holds every fragment in the lane order of the MFMA operand, so no
//   reshuffle is needed on either path.  The activation tile goes through LDS, in
//   a ring of stages filled by direct-to-LDS buffer loads together with the step's
//   block scale bytes.
// * Persistent: one workgroup per CU walks its share of the tiles, and the loads
//   run ahead across tile boundaries, so the next tile's first steps are in flight
//   while the current tile's epilogue runs.
// * Activation fragments are read from LDS into registers ahead of their MFMAs: one
//   half-step ahead (two buffers), or, for the FP4 kernels with every weight group
//   in registers, two half-steps ahead (three buffers), so that no MFMA waits for
//   LDS data.
// * Every half-step issues the same number of memory operations, so each wait is a
//   constant count of outstanding operations, and the workgroup barrier carries no
//   memory fence (the kernel orders its LDS accesses itself).
// * Raw buffer loads return zeros past the end of a tensor, which clips ragged M
//   and padded rows without branches; stores are predicated per row and column.
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "common.hpp"

namespace ditq {
namespace {

constexpr int kRowBytes = 64;    // operand bytes per row per k-step
// Weight row groups per wave staged through LDS on the 2 x 2 grid (measured best):
// FP4 and FP8 split the four evenly (FP8 with all four in registers spills in the
// QK-RMSNorm and gated-residual epilogues and measured 1-3 % slower); MXFP8, whose
// 4 KB groups per k-step the LDS copies do not cover, loads all of them into
// registers.
constexpr int wlds_for(int fmt) { return fmt == FMT_FP4 || fmt == FMT_FP8 ? 2 : 0; }
// Tile-order group height (in M tiles).  8 and 4 run at the same speed on the
// headline shape; 8 keeps each weight tile shared by more of the tiles in flight on
// an XCD, which cuts the L2 miss traffic per launch from 226 to 204 MB (12 and 24
// measured slower).
constexpr int kGroupM = 8;

// WLDS: how many of the wave's 4 weight row groups come through LDS (shared by the
// two waves of a row band, one copy per workgroup); the other TN - WLDS groups are
// loaded straight into registers.  RING: length of that register ring in units (a
// unit = one 64-K MFMA step); unit u is loaded RING-1 units before it is used.
// HD: head_dim of the QK-RMSNorm epilogue (0 otherwise).  WL: waves along N: 2 (a
// 2 x 2 grid, each wave 128 features x BM/2 tokens) or 4 (a 4 x 1 grid, each wave 64
// features x all BM tokens: no weight row is needed by two waves, so all weights go
// straight to registers and only the activation tile is shared).
// F32: the debug form of the kernel, whose store writes the fp32 value the bf16 store
// would round (a separate instantiation, so that the production kernels carry no
// trace of it).
// FB: activation fragment buffers in registers.  2: each half-step reads the fragments
// the next half-step consumes.  3 (the block-scaled formats): each half-step reads the
// fragments consumed two half-steps later, so no MFMA waits for LDS data.
template <int FMT_, int EPI_, int TM_, int RING_, int WLDS_, int HD_ = 0, int WL_ = 2, bool F32_ = false,
          int FB_ = 2>
struct Tile {
  static constexpr int FMT = FMT_, EPI = EPI_, TM = TM_, RING = RING_, WLDS = WLDS_, HD = HD_, FB = FB_;
  static constexpr bool F32 = F32_;
  using Debug = Tile<FMT_, EPI_, TM_, RING_, WLDS_, HD_, WL_, true, FB_>;
  static constexpr int WAVES_N = WL_, WAVES_M = 4 / WL_, TN = 8 / WL_, NW = 4, NT = 256;
  static constexpr int WN = 32 * TN, WM = 32 * TM;
  static constexpr int BN = WN * WAVES_N, BM = WM * WAVES_M;
  static constexpr bool MX = FMT != FMT_FP8;                   // E8M0 block scales applied by the MFMA
  static constexpr int CH = MX ? 2 : 1;                        // units per k-step
  static constexpr int KSTEP = 64 * CH;
  static constexpr bool NV = FMT == FMT_NV4;                   // E4M3 block-16 scales, dequantized in registers
  static constexpr int FRAG = is_fp4_codes(FMT) ? 1024 : 2048; // bytes of one 32x64 operand fragment
  static constexpr int FRAG_LOADS = FRAG / 1024;               // 16-byte loads per lane per fragment
  static constexpr int MFMA_PER_UNIT = NV ? 4 : 1;             // MFMAs per result tile and 64-K unit
  static constexpr int APANELS = FMT == FMT_MX8 ? 2 : 1;       // 64-byte activation code panels per k-step
  // E8M0 scales on the 4 x 1 grid: one 1 KB scale copy per wave and stage (activation
  // or weight scales by wave parity) instead of two 256-byte ones; measured ~1 %
  // faster there, and neutral to slower on the 2 x 2 grid
  static constexpr bool SC1 = MX && !NV && WL_ == 4;
  static constexpr int TND = TN - WLDS;                        // weight groups loaded into registers
  // The cursors' tile changes (once per tile in a k-loop of 24+ half-steps) laid out
  // as cold code, so that the k-loop runs straight through without taken branches.
  // Same-box A/B on three boxes, outputs identical: the FP4 gated-SiLU kernel with
  // three fragment buffers 1.2 % faster (117.2 -> 115.8, 114.6 -> 113.7, 121.8 ->
  // 120.4 us); the identity and GELU kernels of that family 1-2 % slower, FP4
  // QK-RMSNorm head_dim 128 0.4 % slower (93.4 -> 93.8 us), and in the other kernels
  // the changed layout moves register allocation (QK-RMSNorm with 256-token tiles:
  // 0 -> 14-16 spilled VGPRs), so they keep the default layout.
  static constexpr bool COLD_WRAP = FB_ == 3 && EPI == EPI_GATED_SILU;
  static constexpr int UNIT_LOADS = TND * FRAG_LOADS;
  // k-steps per unrolled group: whole turns of the weight ring (and, with three fragment
  // buffers, of those too: lcm(RING, 3) units)
  static constexpr int STEPS_PER_GROUP = FB == 3 ? (RING % 3 == 0 ? RING : 3 * RING) / CH : RING / CH;
  static constexpr int GROUP_BYTES = FRAG * CH;                // one 32-row group per k-step (2 KB)
  // LDS stage: weight codes of the LDS groups | activation codes | activation scale
  // words | weight scale records
  static constexpr int W_BYTES = WAVES_N * WLDS * GROUP_BYTES;
  static constexpr int A_OFF = W_BYTES;
  static constexpr int A_BYTES = BM * kRowBytes * APANELS;
  static constexpr int AS_OFF = A_OFF + A_BYTES;
  // scale bytes per token / per 32-row group and 128-K step: E8M0 4 / 128, NVFP4 8 / 256
  static constexpr int AS_BYTES = NV ? (6 * BM + 1024 + 255) / 256 * 256
                                : SC1 ? 1024 : MX ? (3 * BM + 256 + 255) / 256 * 256 : 0;
  static constexpr int WS_OFF = AS_OFF + AS_BYTES;
  static constexpr int WS_BYTES = NV ? BN / 32 * 256 : MX ? BN / 32 * 128 : 0;
  static constexpr int STAGE = (WS_OFF + WS_BYTES + 255) / 256 * 256;
  // QK-RMSNorm: waves along N per head (a head wider than one wave's columns sums
  // its squares across waves through LDS: WAVES_N x BM per-token partial sums)
  static constexpr int HEAD_WAVES = HD > WN ? HD / WN : 1;
  static constexpr int RED_BYTES = HEAD_WAVES > 1 ? WAVES_N * BM * 4 : 0;
  static constexpr int STAGES_FIT = (160 * 1024 - 1024 - RED_BYTES) / STAGE;
  static constexpr int WCK = W_BYTES / 1024 / NW;            // 1 KB weight copies per wave per stage
  static constexpr int ACK = A_BYTES / 1024 / NW;            // 1 KB activation copies per wave per stage
  static constexpr int ACKP = ACK / APANELS;                   // ... per code panel
  static constexpr int NCOPY = WCK + ACK + (SC1 ? 1 : MX ? 2 : 0);  // + activation / weight scale copies
  // Memory operations every wave issues per half-step: FP4 / MXFP8 load one unit
  // per half and copy a stage in the second half; FP8 does both in the second half.
  static constexpr int OPS_H0 = MX ? UNIT_LOADS : 0;
  static constexpr int OPS_H1 = NCOPY + UNIT_LOADS;
  static constexpr int OPS_STEP = OPS_H0 + OPS_H1;
  // Ring depth: at most 5 stages, as many as fit in LDS, and few enough that the
  // wait for a stage stays within vmcnt's range (63 operations in flight).
  static constexpr int STAGES_VM = (63 - OPS_H0) / OPS_STEP + 2;
  static constexpr int STAGES_CAP = FB == 3 ? 6 : 5;          // three buffers read a stage one step earlier
  static constexpr int STAGES = STAGES_FIT < STAGES_CAP ? (STAGES_FIT < STAGES_VM ? STAGES_FIT : STAGES_VM)
                                                        : (STAGES_CAP < STAGES_VM ? STAGES_CAP : STAGES_VM);
  static constexpr int JUNK_OFF = STAGES * STAGE;            // target of the prologue's padding copies
  static constexpr int RED_OFF = JUNK_OFF + 1024;            // per-token partial sums of squares
  static constexpr int LDS_BYTES = RED_OFF + RED_BYTES;
  // Waits, as the number of operations that may stay outstanding (vmcnt counts
  // in issue order; the counts below hold whatever the order inside a half).
  //   unit u used in half h: issued in half h - (RING - 1), so the RING - 2 halves
  //   in between were all issued after it (FP8: units are steps, issued in the
  //   second half of step g - (RING - 1)).
  static constexpr int WAIT_UNIT = MX ? (RING - 2) / 2 * OPS_STEP : (RING - 2) * OPS_H1;
  //   stage g+1 (needed at the barrier of step g): issued in the second half of
  //   step g + 1 - STAGES; steps g+2-STAGES .. g-1 and the first half of g follow.
  //   With three fragment buffers stage g+2 (read from the next step on): one step less.
  static constexpr int WAIT_STAGE = (STAGES - (FB == 3 ? 3 : 2)) * OPS_STEP + OPS_H0;
  static constexpr int WAIT_BARRIER = MX ? (WAIT_UNIT < WAIT_STAGE ? WAIT_UNIT : WAIT_STAGE) : WAIT_STAGE;
  // prologue: the half-steps before step 0 that issue stage 0 .. STAGES-1 and unit 0 .. RING-2
  static constexpr int PRO_HALVES = MX ? (2 * STAGES - 1 > RING - 1 ? 2 * STAGES - 1 : RING - 1)
                                       : 2 * (STAGES > RING - 1 ? STAGES : RING - 1);
  static_assert(A_BYTES == ACK * 1024 * NW && W_BYTES == WCK * 1024 * NW, "whole 1 KB copies per wave");
  static_assert(WLDS >= 0 && WLDS <= TN, "weight groups split between LDS and registers");
  static_assert(NV ? 6 * BM + 1024 <= AS_BYTES && 8 * BM <= 6 * BM + 1024 && WS_BYTES == 2048
                   : SC1 ? 4 * BM <= AS_BYTES && WS_BYTES == 1024 : 3 * BM + 256 <= AS_BYTES || !MX,
                "overlapping scale copies fit and cover the tile");
  static_assert(ACK % APANELS == 0, "whole activation copies per panel");
  static_assert(WLDS == 0 || GROUP_BYTES == 2048, "LDS weight groups are copied as two 1 KB halves");
  static_assert(RING % CH == 0 && RING >= 4, "ring holds whole k-steps");
  static_assert(FB == 2 || (FB == 3 && MX), "three fragment buffers: the two-unit k-step of the block-scaled path");
  static_assert(WAIT_UNIT < 64 && WAIT_STAGE < 64, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024 && STAGES >= 3, "LDS");
  static_assert(TN * TM * 16 <= 256, "accumulators fit in the AGPRs");
  static_assert((WAVES_N == 2 || (WAVES_N == 4 && WLDS == 0)) && (EPI != EPI_GATED_SILU || TN % 2 == 0),
                "a 4 x 1 grid shares no weights; a wave holds whole gate/up pairs");
};

struct Params {
  const uint8_t* a_codes;
  const void* a_scales;       // FP4 / MXFP8: E8M0 u8 [M][K/32]; FP8: f32 [M]
  const uint8_t* w_codes;     // blob + header
  const void* w_scales;       // FP4 / MXFP8: E8M0 records; FP8: f32 [Np]
  uint16_t* out;              // bf16 output, or null when only the quantized output is wanted
  float* out_f32;             // debug: the fp32 values the bf16 store would round, instead of it (or null)
  uint8_t* q_codes;           // FP4 quantization of the output for the next GEMM, or null
  uint8_t* q_scales;
  int M, N, K, ldo;
  int tiles_m, tiles_n, tiles;
  const uint16_t* residual;   // gated residual: bf16 [M][ldr] (may be `out`), gate fp32 [..][N]
  const float* gate;
  int ldr, rows_per_gate;
  uint32_t a_bytes, w_bytes, as_bytes, ws_bytes;
  const float* gamma_q;
  const float* gamma_k;
  float eps;
  int n_heads;
  const float* a_tscale;      // NVFP4 tensor scales (device)
  const float* w_tscale;
};

// Activation LDS rows are 64 bytes = 4 chunks of 16 bytes; chunk c of row r is
// stored at slot c ^ swz(r).  For a fixed logical chunk, rows r..r+7 (one 32-bank
// cycle of 16-byte reads) and r..r+15 (one 64-bank cycle) land in distinct banks.
__device__ __host__ constexpr int swz(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// Tile order: kGroupM tiles down M, then across N, group after group; a workgroup
// that sits on XCD x (workgroup id mod 8, the round-robin the dispatcher deals
// ids in) walks a contiguous eighth of that order, so the tiles that are in
// flight on one XCD share operand rows through its L2.
__device__ inline void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
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
//
// With q_codes set, the tile's 32 columns of each token (one E8M0 block) are also
// quantized to FP4 for the next GEMM, in the activation layout dit_quantize_act
// writes: the bf16 values (exactly what the bf16 output holds) get the block
// scale from their largest magnitude, shared by the two partner lanes, and the
// same E2M1 rounding (page "How fal made Ideogram V4 6x faster", paragraph 2;
// page "Versnellende diffusiemodellen met TheStage AI", on-the-fly activation
// scales).  The result equals quantizing the bf16 output, bit for bit.
template <class T>
__device__ inline void store_tile(const Params& p, int row, bool row_ok, int col0, int ncols, int h,
                                  const float* v) {
  if constexpr (T::F32) {
    // debug store: the lane's four runs of 4 columns (8g + 4h) as fp32, no rounding
    if (row_ok) {
      float* o = p.out_f32 + (size_t)row * p.ldo;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = col0 + 8 * g + 4 * h;
        if (c < ncols) *reinterpret_cast<v4f*>(o + c) = v4f{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
      }
    }
    return;
  }
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
  const int c0 = col0 + 8 * h, c1 = col0 + 16 + 8 * h;
  if ((T::FMT != FMT_FP4 || p.out != nullptr) && row_ok) {
    uint16_t* o = p.out + (size_t)row * p.ldo;
    if (c0 < ncols) *reinterpret_cast<v4i*>(o + c0) = v4i{(int)g[0], (int)g[1], (int)g[2], (int)g[3]};
    if (c1 < ncols) *reinterpret_cast<v4i*>(o + c1) = v4i{(int)g[4], (int)g[5], (int)g[6], (int)g[7]};
  }
  if (T::FMT == FMT_FP4 && p.q_codes != nullptr) {
    const v4i r0 = {(int)g[0], (int)g[1], (int)g[2], (int)g[3]};
    const v4i r1 = {(int)g[4], (int)g[5], (int)g[6], (int)g[7]};
    uint32_t m = max(absmax8(r0), absmax8(r1));
    // permlane32_swap(m, m) gives lanes 32..63 their partner's m in element 0 and
    // lanes 0..31 theirs in element 1 (the other element is the lane's own m)
    const auto mm = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    m = max(m, max((uint32_t)mm[0], (uint32_t)mm[1]));
    const uint32_t byte = fp4_scale_byte(m);
    const uint32_t q0 = fp4_encode8(r0, byte), q1 = fp4_encode8(r1, byte);
    if (row_ok && col0 < ncols) {
      // K-panel-major: panel col/128, byte (col % 128) / 2 of the token's 64-byte row;
      // the scale byte of block col/32 at byte (col / 32) % 4 of its 4-byte row
      const size_t prow = (size_t)(col0 >> 7) * p.M + row;
      *reinterpret_cast<uint32_t*>(p.q_codes + prow * 64 + ((c0 & 127) >> 1)) = q0;
      *reinterpret_cast<uint32_t*>(p.q_codes + prow * 64 + ((c1 & 127) >> 1)) = q1;
      if (h == 0) p.q_scales[prow * 4 + ((col0 >> 5) & 3)] = (uint8_t)byte;
    }
  }
}

// SiLU(x) = x / (1 + e^-x) with the hardware exp2 and reciprocal (about 1 ulp
// each).  For very negative x, e^-x = inf and the result is -0, never NaN.
__device__ inline float silu(float x) {
  const float e = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}


// GELU, tanh form: 0.5 x (1 + tanh(u)) = x / (1 + e^(-2u)), u = sqrt(2/pi) (x +
// 0.044715 x^3), with the hardware exp2 and reciprocal.  Saturates to x and -0
// without NaN (an infinite e^(-2u) gives x * 0).
__device__ inline float gelu_tanh(float x) {
  const float t = x * (1.0f + 0.044715f * x * x);                  // u / sqrt(2/pi)
  const float e = __builtin_amdgcn_exp2f(-2.3022081981443250f * t);  // e^(-2u) = 2^(-2 sqrt(2/pi) log2(e) t)
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// The same for the 16 values of a result tile, in stages (all exponentials, then all
// reciprocals, then the products) held apart by scheduling barriers: the 16 chains
// are independent, and issued one after another each would wait on its own
// transcendental results.  Same operations and rounding as silu / gelu_tanh.
__device__ __forceinline__ void silu_mul16(const float* g, const float* u, float* v) {
  float e[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(-g[r] * 1.4426950408889634f);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_rcpf(1.0f + e[r]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = g[r] * e[r] * u[r];
}
__device__ __forceinline__ void gelu_tanh16(float* v) {
  float e[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(-2.3022081981443250f * (v[r] * (1.0f + 0.044715f * v[r] * v[r])));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_rcpf(1.0f + e[r]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = v[r] * e[r];
}

// ---------------------------------------------------------------- operands
// Activation fragments of one unit (TM token tiles): lane L holds token row
// wm*WM + 32*tm + L%32 (FP4: the 16 bytes of K chunk 32*(L/32), logical chunk
// 2J + L/32 of the 64-byte row; FP8: two 16-byte runs, logical chunks L/32 and
// 2 + L/32 of the row, in the 8-bit operand order of the MFMA; MXFP8: the same
// two runs of code panel J).
template <class T>
struct AFrag {
  v4i a[T::TM][T::FRAG_LOADS];
  v4i w[T::WLDS > 0 ? T::WLDS : 1][T::FRAG_LOADS];   // weight groups read from LDS
};

template <class T, int J>
__device__ __forceinline__ void load_act(AFrag<T>& f, const uint8_t* stage, int wn, int wm, int lane) {
  const int h = lane >> 5, l32 = lane & 31;
  // weight fragments of the LDS groups: copied verbatim from the blob (lane order)
#pragma unroll
  for (int g = 0; g < T::WLDS; ++g)
#pragma unroll
    for (int l = 0; l < T::FRAG_LOADS; ++l)
      f.w[g][l] = *reinterpret_cast<const v4i*>(stage + (wn * T::WLDS + g) * T::GROUP_BYTES + J * T::FRAG +
                                                (T::FRAG / 64) * lane + 16 * l);
  stage += T::A_OFF;
#pragma unroll
  for (int tm = 0; tm < T::TM; ++tm) {
    const int r = wm * T::WM + 32 * tm + l32;
    const uint8_t* row = stage + r * kRowBytes;
    if constexpr (is_fp4_codes(T::FMT)) {
      f.a[tm][0] = *reinterpret_cast<const v4i*>(row + 16 * ((2 * J + h) ^ swz(r)));
    } else {
      // 8-bit operands: the MFMA takes k = 16h .. 16h+15 in its first four registers
      // and k = 32 + 16h .. in the other four (logical chunks h and 2 + h)
      const uint8_t* prow = row + J * T::BM * kRowBytes;      // MXFP8: unit J's panel (FP8: J = 0)
      f.a[tm][0] = *reinterpret_cast<const v4i*>(prow + 16 * (h ^ swz(r)));
      f.a[tm][1] = *reinterpret_cast<const v4i*>(prow + 16 * ((2 + h) ^ swz(r)));
    }
  }
}

// Weight fragments of one unit, straight from the blob into registers.
template <class T>
struct WUnit {
  v4i w[T::TND > 0 ? T::TND : 1][T::FRAG_LOADS];
};

// Scale words of one k-step (FP4, MXFP8): a weight record's 16-bit word per lane holds the
// bytes of units J = 0, 1; two row groups share a register (group tn in bytes
// 2*(tn%2) + J, picked by op_sel).  A token's 4 scale bytes are its blocks 0..3 of
// the step, and this lane's units J = 0, 1 take blocks 2J + h (selector byte 0x0C
// gives a zero byte).
// NVFP4: a weight word holds the lane's four E4M3 bytes of the k-step (unit J, block
// b at byte 2J + b); an activation word the token's four bytes for this lane group.
template <class T>
struct Scales {
  uint32_t w[T::NV ? T::TN : T::TN / 2];
  uint32_t a[T::TM];
};

template <class T>
__device__ __forceinline__ void load_scales(Scales<T>& sc, const uint8_t* stage, int wn, int wm, int lane) {
  if constexpr (T::NV) {
    const int l32 = lane & 31;
    // the token's 8 bytes are blocks 0..7 of the step; this lane group takes blocks
    // 4J + 2h + b, i.e. bytes (2h, 2h+1, 4+2h, 5+2h)
    const uint32_t sel = (lane & 32) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn)
      sc.w[tn] = *reinterpret_cast<const uint32_t*>(stage + T::WS_OFF + (wn * T::TN + tn) * 256 + 4 * lane);
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
      const uint2 v = *reinterpret_cast<const uint2*>(stage + T::AS_OFF + 8 * (wm * T::WM + 32 * tm + l32));
      sc.a[tm] = __builtin_amdgcn_perm(v.y, v.x, sel);
    }
  } else if constexpr (T::MX) {
    const int l32 = lane & 31;
#pragma unroll
    for (int t2 = 0; t2 < T::TN / 2; ++t2) {
      const uint8_t* rec = stage + T::WS_OFF + (wn * T::TN + 2 * t2) * 128 + 2 * lane;
      sc.w[t2] = (uint32_t)*reinterpret_cast<const uint16_t*>(rec) |
                 ((uint32_t)*reinterpret_cast<const uint16_t*>(rec + 128) << 16);
    }
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm)
      sc.a[tm] = *reinterpret_cast<const uint32_t*>(stage + T::AS_OFF + 4 * (wm * T::WM + 32 * tm + l32));
  }
}

template <class T>
__device__ __forceinline__ void select_scales(Scales<T>& sc, int lane) {
  if constexpr (T::MX && !T::NV) {
    const uint32_t sel = (lane & 32) ? 0x0C0C0301u : 0x0C0C0200u;
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) sc.a[tm] = __builtin_amdgcn_perm(0u, sc.a[tm], sel);
  }
}

// MFMAs of unit J (op_sel byte of the block scales) over token tiles [TM0, TM1); ZERO starts the
// sums from 0 (first step of a tile) instead of the accumulators.
template <class T>
__device__ __forceinline__ v8i operand(const v4i (&x)[T::FRAG_LOADS]) {
  if constexpr (T::FMT == FMT_FP4)
    return __builtin_shufflevector(x[0], x[0], 0, 1, 2, 3, -1, -1, -1, -1);
  else
    return __builtin_shufflevector(x[0], x[T::FRAG_LOADS - 1], 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// NVFP4: eight E2M1 codes (one dword) times an f16 block scale -> eight f16 (exact).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x8 nv4_dequant8(uint32_t codes, _Float16 s) {
  const f16x2 ss = {s, s};
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
__device__ __forceinline__ _Float16 nv4_scale(uint32_t word, int byte) {
  return (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)(word >> (8 * byte)), 0);
}

template <class T, int J, int TM0, int TM1, bool ZERO>
__device__ __forceinline__ void mfma_part(v16f (&acc)[T::TN][T::TM], const WUnit<T>& wu, const AFrag<T>& f,
                                          const Scales<T>& sc) {
  if constexpr (T::NV) {
    // Sub-step i takes dword i of every fragment (codes 8i .. 8i+7 of the lane, block
    // i/2): A and B lanes pair element by element, so any lane-local K order shared
    // by both operands gives the same dot product.
    static_for<0, 4>([&](auto i_c) __attribute__((always_inline)) {
      constexpr int i = decltype(i_c)::value, b = i / 2;
      f16x8 wv[T::TN], av[T::TM];
#pragma unroll
      for (int tn = 0; tn < T::TN; ++tn) {
        const v4i x = tn < T::WLDS ? f.w[tn < T::WLDS ? tn : 0][0] : wu.w[tn >= T::WLDS ? tn - T::WLDS : 0][0];
        wv[tn] = nv4_dequant8((uint32_t)x[i], nv4_scale(sc.w[tn], 2 * J + b));
      }
#pragma unroll
      for (int tm = TM0; tm < TM1; ++tm) av[tm] = nv4_dequant8((uint32_t)f.a[tm][0][i], nv4_scale(sc.a[tm], 2 * J + b));
#pragma unroll
      for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
        for (int tm = TM0; tm < TM1; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wv[tn], av[tm], (ZERO && i == 0) ? v16f{} : acc[tn][tm],
                                                                0, 0, 0);
    });
    return;
  }
  static_for<0, T::TN>([&](auto tn_c) __attribute__((always_inline)) {
    constexpr int tn = decltype(tn_c)::value;
    v8i w;
    if constexpr (tn < T::WLDS)
      w = operand<T>(f.w[tn]);
    else
      w = operand<T>(wu.w[tn - T::WLDS]);
#pragma unroll
    for (int tm = TM0; tm < TM1; ++tm) {
      const v16f c = ZERO ? v16f{} : acc[tn][tm];
      if constexpr (T::FMT == FMT_FP4)
        acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            w, operand<T>(f.a[tm]), c, 4, 4, 2 * (tn & 1) + J, (int)sc.w[tn / 2], J, (int)sc.a[tm]);
      else if constexpr (T::FMT == FMT_MX8)
        acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            w, operand<T>(f.a[tm]), c, 0, 0, 2 * (tn & 1) + J, (int)sc.w[tn / 2], J, (int)sc.a[tm]);
      else
        acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, operand<T>(f.a[tm]), c, 0, 0, 0,
                                                                      0x7F7F7F7F, 0, 0x7F7F7F7F);
    }
  });
}

// Order of the current scheduling region: LDS reads first, then the MFMAs with
// the NV vector-memory operations spread evenly between them.
template <int NM, int NV>
__device__ __forceinline__ void spread_vmem() {
  constexpr int kDsRead = 0x100, kMfma = 0x008, kVmem = 0x010;
  __builtin_amdgcn_sched_group_barrier(kDsRead, 64, 0);
  if constexpr (NV == 0) {
    __builtin_amdgcn_sched_group_barrier(kMfma, NM, 0);
  } else {
    // memory operation i follows MFMA number floor((i + 1) * NM / (NV + 1)): evenly
    // spaced over the whole half-step (the four waves issue in step, so bunching the
    // operations would ask the CU's vector memory path for several KB at once)
    static_for<0, NV>([&](auto i_c) __attribute__((always_inline)) {
      constexpr int i = decltype(i_c)::value;
      constexpr int before = (i + 1) * NM / (NV + 1) - i * NM / (NV + 1);
      if constexpr (before > 0) __builtin_amdgcn_sched_group_barrier(kMfma, before, 0);
      __builtin_amdgcn_sched_group_barrier(kVmem, 1, 0);
    });
    constexpr int rest = NM - NV * NM / (NV + 1);
    if constexpr (rest > 0) __builtin_amdgcn_sched_group_barrier(kMfma, rest, 0);
  }
}

// ---------------------------------------------------------------- epilogues
__device__ __forceinline__ void barrier();
__device__ __forceinline__ void wait_lds();

// The small op and the store of one 32 x 32 result tile of the identity and GELU
// epilogues (v: its values, row and column scales applied), for the FP8
// row/column-scale path.  A separate function on purpose: written inline, or used
// by the other kernels' epilogue loop, it changes their register allocation (FP8
// identity and GELU spill 3 VGPRs more; FP4 GELU measured 0.4 % slower).
template <class T>
__device__ __forceinline__ void finish_tile(const Params& p, float (&v)[16], int tn, int row, bool ok, int n0w,
                                            int h) {
  static_assert(T::EPI == EPI_IDENTITY || T::EPI == EPI_GELU_TANH, "identity and GELU only");
  if constexpr (T::EPI == EPI_GELU_TANH) {
    gelu_tanh16(v);
  }
  store_tile<T>(p, row, ok, n0w + 32 * tn, p.N, h, v);
}

template <class T>
__device__ __forceinline__ void epilogue(const Params& p, v16f (&acc)[T::TN][T::TM], int n0w, int m0w, int lane,
                                         int wn, int wm, uint8_t* lds) {
  const int h = lane >> 5, l32 = lane & 31;
  if constexpr (T::NV) {
    // the two tensor scales, before any small op
    const float ts = *p.a_tscale * *p.w_tscale;
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tn][tm][r] *= ts;
  }
  if constexpr (T::FMT == FMT_FP8 && (T::EPI == EPI_IDENTITY || T::EPI == EPI_GELU_TANH)) {
    // result tile outer: the column scales of a result tile are loaded once and
    // serve every token tile (each load waits, on the in-order vector memory
    // counter, for every older load, the next tile's operands included).
    // Same-box A/B, outputs identical: CFG-pair identity 304.9 -> 294.6 us, GELU
    // 175.7 -> 172.5 us.  (The gated residual keeps the order below: this one
    // raises its spills from 1 to 9 VGPRs.)
    float sa[T::TM];
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
      const int row = m0w + 32 * tm + l32;
      sa[tm] = reinterpret_cast<const float*>(p.a_scales)[row < p.M ? row : p.M - 1];
    }
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn) {
      __builtin_amdgcn_sched_barrier(0);
      v4f sw[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        sw[g] = *reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(p.w_scales) + n0w + 32 * tn + 8 * g +
                                              4 * h);
#pragma unroll
      for (int tm = 0; tm < T::TM; ++tm) {
        const int row = m0w + 32 * tm + l32;
        float v[16];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * g + i] = acc[tn][tm][4 * g + i] * (sa[tm] * sw[g][i]);
        finish_tile<T>(p, v, tn, row, row < p.M, n0w, h);
      }
    }
  } else if constexpr (T::FMT == FMT_FP8 && T::EPI == EPI_GATED_SILU) {
    // gate/up result tile pair outer, like the identity / GELU path above.  Same-box
    // A/B, outputs identical: CFG pair 305.4 -> 286.0 us, 4608 x 16384 x 3072
    // 204.9 -> 193.3 us.
    float sa[T::TM];
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
      const int row = m0w + 32 * tm + l32;
      sa[tm] = reinterpret_cast<const float*>(p.a_scales)[row < p.M ? row : p.M - 1];
    }
#pragma unroll
    for (int q = 0; q < T::TN / 2; ++q) {
      __builtin_amdgcn_sched_barrier(0);
      v4f sg[4], su[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float* ws = reinterpret_cast<const float*>(p.w_scales) + n0w + 64 * q + 8 * g + 4 * h;
        sg[g] = *reinterpret_cast<const v4f*>(ws);
        su[g] = *reinterpret_cast<const v4f*>(ws + 32);
      }
#pragma unroll
      for (int tm = 0; tm < T::TM; ++tm) {
        const int row = m0w + 32 * tm + l32;
        float gate[16], up[16], v[16];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            gate[4 * g + i] = acc[2 * q][tm][4 * g + i] * (sa[tm] * sg[g][i]);
            up[4 * g + i] = acc[2 * q + 1][tm][4 * g + i] * (sa[tm] * su[g][i]);
          }
        silu_mul16(gate, up, v);
        store_tile<T>(p, row, row < p.M, n0w / 2 + 32 * q, p.N / 2, h, v);
      }
    }
  } else if constexpr (T::EPI != EPI_QK_RMSNORM) {
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
      __builtin_amdgcn_sched_barrier(0);     // one token tile at a time keeps register use low
      const int row = m0w + 32 * tm + l32;
      const bool ok = row < p.M;
      float sa = 1.0f;
      if constexpr (T::FMT == FMT_FP8) sa = reinterpret_cast<const float*>(p.a_scales)[ok ? row : p.M - 1];
      if constexpr (T::EPI != EPI_GATED_SILU) {
#pragma unroll
        for (int tn = 0; tn < T::TN; ++tn) {
          __builtin_amdgcn_sched_barrier(0);   // one result tile at a time
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
          if constexpr (T::EPI == EPI_GELU_TANH) {
            gelu_tanh16(v);
          }
          if constexpr (T::EPI == EPI_GATE_RESIDUAL) {
            // this lane's 16 columns are 4 runs of 4 (n0 + 8g + 4h + i): the residual
            // as four 8-byte reads, the gate row of the token's sample as four 16-byte
            // reads.  Rows past M read row M - 1, and a 32-column result tile at or past
            // N (the padding of the last tile; N is a multiple of 64, so a tile is
            // wholly in or out) reads nothing: every read stays inside residual[M][ldr]
            // and gate[ceil(M / rows_per_gate)][N], and neither kind of result is
            // stored.  The test is uniform over the wave: a per-lane test measured dozens
            // of register spills more.  The 4-bit formats skip the reads of such a tile,
            // the 8-bit ones read the last 32 columns instead (each form is the one that
            // spills fewer registers in that format's kernels).
            const int rr = ok ? row : p.M - 1;
            constexpr bool kSkip = is_fp4_codes(T::FMT);
            const bool live = kSkip ? n0w + 32 * tn < p.N : true;
            const int col = (kSkip ? n0w + 32 * tn : __builtin_amdgcn_readfirstlane(min(n0w + 32 * tn, p.N - 32))) +
                            4 * h;
            const uint16_t* rp = p.residual + (size_t)rr * p.ldr + col;
            const float* gp = p.gate + (size_t)(rr / p.rows_per_gate) * p.N + col;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              uint2 rv = {0u, 0u};
              v4f gv = {0.0f, 0.0f, 0.0f, 0.0f};
              if (live) {
                rv = *reinterpret_cast<const uint2*>(rp + 8 * g);
                gv = *reinterpret_cast<const v4f*>(gp + 8 * g);
              }
              v[4 * g + 0] = __builtin_fmaf(gv[0], v[4 * g + 0], bf16_lo(rv.x));
              v[4 * g + 1] = __builtin_fmaf(gv[1], v[4 * g + 1], bf16_hi(rv.x));
              v[4 * g + 2] = __builtin_fmaf(gv[2], v[4 * g + 2], bf16_lo(rv.y));
              v[4 * g + 3] = __builtin_fmaf(gv[3], v[4 * g + 3], bf16_hi(rv.y));
            }
          }
          store_tile<T>(p, row, ok, n0w + 32 * tn, p.N, h, v);
        }
      } else {
#pragma unroll
        for (int q = 0; q < T::TN / 2; ++q) {
          __builtin_amdgcn_sched_barrier(0);   // one gate/up pair at a time
          float gate[16], up[16], v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            gate[r] = acc[2 * q][tm][r];
            up[r] = acc[2 * q + 1][tm][r];
          }
          silu_mul16(gate, up, v);
          store_tile<T>(p, row, ok, n0w / 2 + 32 * q, p.N / 2, h, v);
        }
      }
    }
  } else {
    // Per-head QK-RMSNorm.  A head is HW = head_dim / (the wave's columns) waves
    // wide: one wave (2 x 2 grid, head_dim 128), two (2 x 2 grid with head_dim 256,
    // 4 x 1 grid with 128) or four (4 x 1 grid, 256).  Waves of one head exchange
    // per-token partial sums of squares through LDS, and all of them form the same
    // sum (two waves: own + partner; more: the partial sums in one fixed order).
    constexpr int D = T::HD, HW = T::HEAD_WAVES;
    static_assert(D % T::WN == 0, "a head is whole waves wide");
    static_assert(T::BN % D == 0, "a tile holds whole heads");
    if constexpr (T::FMT == FMT_FP8) {
      // the row / column scales first: the norm is taken over the scaled values
      // (result tile outer: a column-scale load serves every token tile)
      float sa[T::TM];
#pragma unroll
      for (int tm = 0; tm < T::TM; ++tm) {
        const int row = m0w + 32 * tm + l32;
        sa[tm] = reinterpret_cast<const float*>(p.a_scales)[row < p.M ? row : p.M - 1];
      }
#pragma unroll
      for (int tn = 0; tn < T::TN; ++tn) {
        v4f sw[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
          sw[g] = *reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(p.w_scales) + n0w + 32 * tn + 8 * g +
                                                4 * h);
#pragma unroll
        for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[tn][tm][4 * g + i] *= sa[tm] * sw[g][i];
      }
    }
    const int part = (n0w / D) / p.n_heads;     // 0 = Q, 1 = K, 2 = V, 3 = padding past N
    auto store_raw = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int tm = 0; tm < T::TM; ++tm) {
        __builtin_amdgcn_sched_barrier(0);
        const int row = m0w + 32 * tm + l32;
#pragma unroll
        for (int tn = 0; tn < T::TN; ++tn) {
          float v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = acc[tn][tm][r];
          store_tile<T>(p, row, row < p.M, n0w + 32 * tn, p.N, h, v);
        }
      }
    };
    // Where every wave of the workgroup has the same part (a head is one wave, or the
    // whole tile), V and padding leave here; otherwise only after the exchange,
    // which every wave of the workgroup must reach.
    constexpr bool uniform_part = HW == 1 || HW == T::WAVES_N;
    if constexpr (uniform_part) {
      if (part >= 3) return;
      if (part == 2) {
        store_raw();
        return;
      }
    }
    const float* gamma = (part == 0 ? p.gamma_q : p.gamma_k) + (wn % HW) * T::WN;
    // Sums of squares per token: the two halves of the wave's columns (the first
    // half's values stay in registers while the second half's sum is formed), then
    // the partner lane's 16 rows of each tile, then the other waves of the head.
    float ss[T::TM];
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
      float ss_first = 0.0f, ss_second = 0.0f;
#pragma unroll
      for (int tn = 0; tn < T::TN / 2; ++tn)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss_first += acc[tn][tm][r] * acc[tn][tm][r];
#pragma unroll
      for (int tn = T::TN / 2; tn < T::TN; ++tn)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss_second += acc[tn][tm][r] * acc[tn][tm][r];
      ss[tm] = ss_first + ss_second;
      ss[tm] += __shfl_xor(ss[tm], 32);
    }
    if constexpr (HW > 1) {
      // every wave still here writes and reaches the barrier
      float* red = reinterpret_cast<float*>(lds + T::RED_OFF);
      if (lane < 32) {
#pragma unroll
        for (int tm = 0; tm < T::TM; ++tm) red[wn * T::BM + wm * T::WM + 32 * tm + l32] = ss[tm];
      }
      wait_lds();
      barrier();
      if constexpr (HW == 2) {
        // own + partner: fp32 addition commutes, so both waves get the same sum
#pragma unroll
        for (int tm = 0; tm < T::TM; ++tm) ss[tm] += red[(wn ^ 1) * T::BM + wm * T::WM + 32 * tm + l32];
      } else {
        const int w0 = wn - wn % HW;
#pragma unroll
        for (int tm = 0; tm < T::TM; ++tm) {
          float sum = 0.0f;
#pragma unroll
          for (int j = 0; j < HW; ++j) sum += red[(w0 + j) * T::BM + wm * T::WM + 32 * tm + l32];
          ss[tm] = sum;
        }
      }
      if constexpr (!uniform_part) {
        if (part >= 3) return;
        if (part == 2) {
          store_raw();
          return;
        }
      }
    }
    float rs[T::TM];
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) rs[tm] = __builtin_amdgcn_rsqf(ss[tm] * (1.0f / D) + p.eps);
    // gamma of a 32-column result tile is loaded once and serves every token tile.
    // Each such load waits, on the in-order vector memory counter, for every older
    // load (the next tile's operands included), so the count of them matters: a
    // third of the loads and waits of the token-tile-outer order.  Same-box A/B,
    // outputs identical, head_dim 128 / 256: FP4 88.9 -> 84.9 / 118.6 -> 111.1 us,
    // FP8 151.0 -> 150.3 / 241.4 -> 231.9, MXFP8 139.7 -> 131.3 / 211.7 -> 206.3,
    // NVFP4 240.6 -> 234.2 / 387.9 -> 379.1.
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      const int t0 = step == 0 ? T::TN / 2 : 0;     // second half first, then revisit the first
#pragma unroll
      for (int tn = t0; tn < t0 + T::TN / 2; ++tn) {
        __builtin_amdgcn_sched_barrier(0);
        v4f gm[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) gm[g] = *reinterpret_cast<const v4f*>(gamma + 32 * tn + 8 * g + 4 * h);
#pragma unroll
        for (int tm = 0; tm < T::TM; ++tm) {
          const int row = m0w + 32 * tm + l32;
          float v[16];
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[4 * g + i] = acc[tn][tm][4 * g + i] * rs[tm] * gm[g][i];
          store_tile<T>(p, row, row < p.M, n0w + 32 * tn, p.N, h, v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- kernel
// An empty volatile asm that reads every accumulator: the MFMAs of a half-step
// must then be issued before it, and it stays ordered with the wait and the barrier
// that follow (MFMAs touch no memory, so without it they may be sunk below the
// barrier).  The asm exists only in the device pass: on the host pass "a" would
// name an x86 register, and the failed constraint would silently drop the kernel's
// host stub.
template <class T>
__device__ __forceinline__ void pin_accumulators(v16f (&acc)[T::TN][T::TM]) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) asm volatile("" ::"a"(acc[tn][tm]));
#endif
}

// One direct-to-LDS copy: lane L fetches BYTES at voff + soff and the hardware
// writes them to dst + BYTES*L.  (A plain device function: inside a lambda the
// builtin would also be compiled for the host, where it fails and takes the
// kernel's host stub with it.)
template <int BYTES>
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, int soff, uint8_t* dst) {
  static_assert(BYTES == 16 || BYTES == 4, "copy width");
  auto* d = (__attribute__((address_space(3))) void*)dst;
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, d, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, d, 4, voff, soff, 0, 0);
}

// The weight fragments of one unit: lane L's FRAG/64 bytes of fragment (group
// tn of the wave's band, unit `unit`), straight into registers; wbase addresses
// the band's first group for this lane, wgroup is the blob stride of a group.
template <class T>
__device__ __forceinline__ void load_unit(WUnit<T>& wu, __amdgpu_buffer_rsrc_t rsrc, uint32_t wbase, int unit,
                                          int wgroup) {
#pragma unroll
  for (int tn = 0; tn < T::TND; ++tn)
#pragma unroll
    for (int l = 0; l < T::FRAG_LOADS; ++l)
      wu.w[tn][l] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(rsrc, wbase, tn * wgroup + unit * T::FRAG + 16 * l, 0));
}

// s_waitcnt vmcnt(n) with the other counters unconstrained, or with lgkmcnt(0)
// as well (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N, bool LDS_TOO = false>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | ((LDS_TOO ? 0x0 : 0xF) << 8) | ((N >> 4) << 14));
}
// s_waitcnt lgkmcnt(0) only
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without a memory fence.  __syncthreads() is also a release
// fence, and with the output stores in the same loop nest the compiler has to
// drain every outstanding memory operation before it, which exposes the latency
// of all the loads in flight on every k-step.  The kernel orders its own memory:
// each wave waits for exactly the operations the barrier protects; the empty asm
// statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <class T>
__global__ void __launch_bounds__(T::NT, 1) gemm_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[T::LDS_BYTES];
  constexpr int S = T::STAGES;
  // readfirstlane: the wave index is uniform, and the compiler must know it (a
  // per-wave buffer descriptor would otherwise become a loop over lanes)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % T::WAVES_N, wm = wave / T::WAVES_N;

  // Persistent schedule: one workgroup per CU.  The XCD of workgroup b (b mod 8)
  // owns a contiguous range of the tile order; its workgroups take every gx-th
  // tile of that range, so the tiles in flight on one XCD stay adjacent.
  const int G = gridDim.x;
  const int X = G < 8 ? G : 8;                     // XCDs that hold workgroups
  const int x = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int gx = (G - x + 7) >> 3;                 // workgroups on this XCD
  const int q = p.tiles / X, r = p.tiles % X;
  const int x0 = x * q + min(x, r), len = q + (x < r ? 1 : 0);
  const int n_mine = jx < len ? (len - jx + gx - 1) / gx : 0;
  if (n_mine == 0) return;                         // uniform over the workgroup
  auto tile_of = [&](int i, int& n0, int& m0) __attribute__((always_inline)) {
    int tmi, tni;
    tile_coords(x0 + jx + (i < n_mine ? i : n_mine - 1) * gx, p.tiles_m, p.tiles_n, tmi, tni);
    n0 = tni * T::BN;
    m0 = tmi * T::BM;
  };

  // k-steps per tile, rounded up to whole unrolled groups of the weight ring.  The
  // steps past K add exact zeros: their activation code and scale offsets lie past
  // the end of those buffers, where raw buffer loads return zeros (the range check
  // covers voffset + soffset), and E2M1 / E4M3 zeros times any finite weight code
  // (the rows that follow in the blob, or zeros past its end) are zero.
  const int nks = (p.K / T::KSTEP + T::STEPS_PER_GROUP - 1) / T::STEPS_PER_GROUP * T::STEPS_PER_GROUP;
  const int units = nks * T::CH;                                  // units per tile
  const uint32_t wgroup = (uint32_t)(p.K / 64) * T::FRAG;         // blob bytes of one 32-row group
  const uint32_t a_panel = (uint32_t)p.M * kRowBytes;            // bytes of one K panel of activation codes
  const auto a_rsrc = make_rsrc(p.a_codes, p.a_bytes);
  const auto w_rsrc = make_rsrc(p.w_codes, p.w_bytes);
  [[maybe_unused]] const auto as_rsrc = make_rsrc(p.a_scales, p.as_bytes);
  [[maybe_unused]] const auto ws_rsrc = make_rsrc(p.w_scales, p.ws_bytes);
  // one 128-K panel of activation scale rows / of weight scale records
  [[maybe_unused]] const uint32_t as_step = (uint32_t)p.M * (T::NV ? 8u : 4u);
  [[maybe_unused]] const uint32_t ws_step = (uint32_t)(padded_rows(p.N) / 32) * (T::NV ? 256u : 128u);

  // Weight cursor: tile and unit that the next weight loads fetch.  Lane L of
  // fragment (group g, unit u) sits at g * wgroup + u * FRAG + L * FRAG/64.
  int wc_i = 0, wc_u = 0;
  uint32_t wbase = 0;
  auto set_w_tile = [&](int i) __attribute__((always_inline)) {
    int n0, m0;
    tile_of(i, n0, m0);
    wbase = (uint32_t)(n0 / 32 + wn * T::TN + T::WLDS) * wgroup + (uint32_t)(T::FRAG / 64) * lane;
  };
  auto advance_w = [&]() __attribute__((always_inline)) {
    const bool wrap = ++wc_u == units;
    if (T::COLD_WRAP ? __builtin_expect(wrap, 0) : wrap) {
      wc_u = 0;
      set_w_tile(++wc_i);
    }
  };
  // Activation cursor: tile and k-step of the next stage.  Activation copy c of
  // wave w = 16 token rows of a K panel (contiguous in the panel-major layout),
  // lane L fetching the logical chunk that the swizzle places at slot L%4 of row
  // 16(w*ACKP + c') + L/4, c' = c mod ACKP in panel c / ACKP (MXFP8 copies two
  // 64-element panels per k-step).  Block-scale copies, 4 bytes per lane: wave w copies the
  // tile's activation scale words from byte w*BM and weight scale records from
  // byte 256w (the activation copies overlap and write the same bytes); on the 4 x 1
  // grid, 16 bytes per lane: an even wave copies the 1 KB from the tile's first
  // activation scale word (BM <= 256 tokens of 4 bytes), an odd wave the tile's 1 KB
  // of weight scale records, waves 2 and 3 repeating waves 0 and 1 so that every wave
  // issues the same operations.  Rows past M read other data; their results are
  // never stored.
  int ac_i = 0, ac_ks = 0;
  uint32_t a_off = 0;
  [[maybe_unused]] uint32_t w_off[T::WCK > 0 ? T::WCK : 1];
  [[maybe_unused]] uint32_t as_off = 0, ws_off = 0;
  [[maybe_unused]] const bool ws_wave = (wave & 1) != 0;         // 4 x 1 grid: the scale copy's source
  [[maybe_unused]] const auto sc_rsrc = ws_wave ? ws_rsrc : as_rsrc;
  [[maybe_unused]] const uint32_t sc_step = ws_wave ? ws_step : as_step;
  [[maybe_unused]] const int sc_dst = ws_wave ? T::WS_OFF : T::AS_OFF;
  auto set_a_tile = [&](int i) __attribute__((always_inline)) {
    int n0, m0;
    tile_of(i, n0, m0);
    // the swizzle of row 16k + L/4 depends on L only, so copy c of the wave is copy 0
    // moved by c * 1 KB
    const int rr = 16 * (wave * T::ACKP) + (lane >> 2);
    a_off = (uint32_t)(m0 + rr) * kRowBytes + 16u * ((lane & 3) ^ swz(rr));
    // weight copy q of the workgroup = half (q % 2) of LDS group q / 2 = group g of
    // row band wn', in the stage's weight area in that order
#pragma unroll
    for (int c = 0; c < T::WCK; ++c) {
      const int q = wave * T::WCK + c, grp = q >> 1;
      const int band = grp / (T::WLDS > 0 ? T::WLDS : 1), g = grp % (T::WLDS > 0 ? T::WLDS : 1);
      w_off[c] = (uint32_t)(n0 / 32 + band * T::TN + g) * wgroup + 1024u * (q & 1) + 16u * lane;
    }
    if constexpr (T::NV) {
      // 16 bytes per lane: wave w copies 1 KB of activation scale rows from byte 2w*BM
      // (overlapping, together the tile's 8*BM bytes) and weight records from byte
      // 1 KB*(w%2) (waves 2, 3 repeat waves 0, 1)
      as_off = (uint32_t)m0 * 8u + (uint32_t)(2 * wave * T::BM) + 16u * lane;
      ws_off = (uint32_t)(n0 / 32) * 256u + 1024u * (wave & 1) + 16u * lane;
    } else if constexpr (T::SC1) {
      as_off = (ws_wave ? (uint32_t)(n0 / 32) * 128u : (uint32_t)m0 * 4u) + 16u * lane;
    } else if constexpr (T::MX) {
      as_off = (uint32_t)m0 * 4u + (uint32_t)(wave * T::BM) + 4u * lane;
      ws_off = (uint32_t)(n0 / 32) * 128u + 256u * wave + 4u * lane;
    }
  };
  auto copy_stage = [&](int slot) __attribute__((always_inline)) {
    uint8_t* base = lds + slot;
#pragma unroll
    for (int c = 0; c < T::WCK; ++c)
      copy_to_lds<16>(w_rsrc, w_off[c], ac_ks * T::GROUP_BYTES, base + (wave * T::WCK + c) * 1024);
#pragma unroll
    for (int c = 0; c < T::ACK; ++c) {
      const int panel = c / T::ACKP, cc = c % T::ACKP;
      copy_to_lds<16>(a_rsrc, a_off, (ac_ks * T::APANELS + panel) * a_panel + cc * 1024,
                      base + T::A_OFF + panel * T::BM * kRowBytes + (wave * T::ACKP + cc) * 1024);
    }
    if constexpr (T::NV) {
      copy_to_lds<16>(as_rsrc, as_off, ac_ks * as_step, base + T::AS_OFF + 2 * wave * T::BM);
      copy_to_lds<16>(ws_rsrc, ws_off, ac_ks * ws_step, base + T::WS_OFF + 1024 * (wave & 1));
    } else if constexpr (T::SC1) {
      copy_to_lds<16>(sc_rsrc, as_off, ac_ks * sc_step, base + sc_dst);
    } else if constexpr (T::MX) {
      copy_to_lds<4>(as_rsrc, as_off, ac_ks * as_step, base + T::AS_OFF + wave * T::BM);
      copy_to_lds<4>(ws_rsrc, ws_off, ac_ks * ws_step, base + T::WS_OFF + 256 * wave);
    }
  };
  auto advance_a = [&]() __attribute__((always_inline)) {
    const bool wrap = ++ac_ks == nks;
    if (T::COLD_WRAP ? __builtin_expect(wrap, 0) : wrap) {
      ac_ks = 0;
      set_a_tile(++ac_i);
    }
  };
  // Copies that only keep the operation count of a prologue half-step uniform.
  auto pad = [&](auto n_c) __attribute__((always_inline)) {
    constexpr int n = decltype(n_c)::value;
#pragma unroll
    for (int i = 0; i < n; ++i) copy_to_lds<16>(a_rsrc, 16u * lane, 0, lds + T::JUNK_OFF);
  };

  WUnit<T> ring[T::RING];
  AFrag<T> fr[T::FB];
  AFrag<T>& fa = fr[0];
  AFrag<T>& fb = fr[1];
  Scales<T> sc, sn;
  v16f acc[T::TN][T::TM];

  // Prologue: the half-steps before step 0, issuing what they would issue in the
  // steady state (stages 0 .. S-1, units 0 .. RING-2), padded where the target
  // does not exist yet.
  set_w_tile(0);
  set_a_tile(0);
  constexpr int PRO = T::PRO_HALVES;
  static_for<0, PRO>([&](auto k_c) __attribute__((always_inline)) {
    constexpr int h = decltype(k_c)::value - PRO;           // half-step index, negative
    constexpr int J = h & 1, g = h >> 1;                     // k-step g (floor), second half if J
    if constexpr (T::MX || J == 1) {
      if constexpr (J == 1) {
        if constexpr (g + S >= 0) {
          copy_stage(((g + S) % S) * T::STAGE);
          advance_a();
        } else {
          pad(std::integral_constant<int, T::NCOPY>{});
        }
      }
      constexpr int u = T::MX ? h + T::RING - 1 : g + T::RING - 1;
      if constexpr (u >= 0) {
        load_unit<T>(ring[u % T::RING], w_rsrc, wbase, wc_u, (int)wgroup);
        advance_w();
      } else {
        pad(std::integral_constant<int, T::UNIT_LOADS>{});
      }
    }
  });
  // Stage 0 went out in the second half of step -S, stage 1 in that of step 1 - S;
  // everything issued after the half of the last stage needed (stage 1 with three
  // fragment buffers, which read both stages before step 0's MFMAs) may still be in
  // flight.
  constexpr int PRO_WAIT = []() {
    int n = 0;
    for (int h = -2 * S + (T::FB == 3 ? 4 : 2); h < 0; ++h) {
      const bool second = (h & 1) != 0;
      n += T::MX ? (second ? T::OPS_H1 : T::OPS_H0) : (second ? T::OPS_H1 : 0);
    }
    return n < 63 ? n : 63;
  }();
  static_assert(2 * S - 1 <= PRO, "the prologue issues stage 0");
  wait_vmcnt<PRO_WAIT>();
  barrier();
  load_scales<T>(sc, lds, wn, wm, lane);
  load_act<T, 0>(fa, lds, wn, wm, lane);
  if constexpr (T::FB == 3) load_act<T, 1>(fb, lds, wn, wm, lane);
  select_scales<T>(sc, lane);

  // One k-step.  Step g computes from LDS slot g mod S (byte offset `cur`) and
  // weight ring slots (units).  The barrier sits between the two halves of the
  // MFMAs: before it every wave has issued the first half (which keeps the matrix
  // core busy through the wait); after it stage g+1 is visible to all waves and
  // slot `cur` is free, so the copy of stage g+S goes there while the second half
  // runs.  Each half issues its LDS reads before its MFMAs, so the fragments
  // being read live in other registers than the ones being consumed; weight loads
  // go into the ring slot consumed one half earlier.  ZERO: the tile's first step,
  // whose MFMAs start from zero.
  int cur = 0;
  auto step = [&](auto si_c, auto zero_c) __attribute__((always_inline)) {
    constexpr int SI = decltype(si_c)::value;
    constexpr bool ZERO = decltype(zero_c)::value;
    const int nxt = cur + T::STAGE == S * T::STAGE ? 0 : cur + T::STAGE;
    if constexpr (T::FB == 3) {
      // unit U = 2 step + J uses fragment buffer U mod 3 and reads unit U + 2's (stage
      // g+1) into buffer (U + 2) mod 3, the one the previous half-step consumed
      constexpr int u0 = (2 * SI) % T::RING, u1 = u0 + 1;
      constexpr int l0 = (u0 + T::RING - 1) % T::RING, l1 = u0;
      constexpr int f0 = (2 * SI) % 3, f1 = (2 * SI + 1) % 3, f2 = (2 * SI + 2) % 3;
      wait_vmcnt<T::WAIT_UNIT>();                  // unit u0 has landed
      __builtin_amdgcn_sched_barrier(0);
      load_scales<T>(sn, lds + nxt, wn, wm, lane);
      load_act<T, 0>(fr[f2], lds + nxt, wn, wm, lane);
      load_unit<T>(ring[l0], w_rsrc, wbase, wc_u, (int)wgroup);
      mfma_part<T, 0, 0, T::TM, ZERO>(acc, ring[u0], fr[f0], sc);
      spread_vmem<T::TN * T::TM * T::MFMA_PER_UNIT, T::UNIT_LOADS>();
      pin_accumulators<T>(acc);
      __builtin_amdgcn_sched_barrier(0);
      advance_w();
      wait_vmcnt<T::WAIT_BARRIER, true>();         // stage g+2 and unit u1 have landed; reads of `cur` done
      barrier();
      __builtin_amdgcn_sched_barrier(0);
      load_act<T, 1>(fr[f0], lds + nxt, wn, wm, lane);   // reads before the copies (see below)
      copy_stage(cur);
      load_unit<T>(ring[l1], w_rsrc, wbase, wc_u, (int)wgroup);
      mfma_part<T, 1, 0, T::TM, false>(acc, ring[u1], fr[f1], sc);
      spread_vmem<T::TN * T::TM * T::MFMA_PER_UNIT, T::NCOPY + T::UNIT_LOADS>();
      pin_accumulators<T>(acc);
      __builtin_amdgcn_sched_barrier(0);
      advance_w();
      advance_a();
      sc = sn;
      select_scales<T>(sc, lane);
    } else if constexpr (T::MX) {
      constexpr int u0 = (2 * SI) % T::RING, u1 = u0 + 1;
      constexpr int l0 = (u0 + T::RING - 1) % T::RING, l1 = u0;
      wait_vmcnt<T::WAIT_UNIT>();                  // unit u0 has landed
      __builtin_amdgcn_sched_barrier(0);
      load_act<T, 1>(fb, lds + cur, wn, wm, lane);
      load_unit<T>(ring[l0], w_rsrc, wbase, wc_u, (int)wgroup);
      mfma_part<T, 0, 0, T::TM, ZERO>(acc, ring[u0], fa, sc);
      spread_vmem<T::TN * T::TM * T::MFMA_PER_UNIT, T::UNIT_LOADS>();
      pin_accumulators<T>(acc);
      __builtin_amdgcn_sched_barrier(0);
      advance_w();
      wait_vmcnt<T::WAIT_BARRIER, true>();         // stage g+1 and unit u1 have landed; reads of `cur` done
      barrier();
      __builtin_amdgcn_sched_barrier(0);
      // The reads of the next stage come first in program order: the copies write
      // LDS, which the compiler cannot tell apart from the slot being read, so copies
      // placed before the reads would be held in front of every MFMA of the half.
      load_scales<T>(sn, lds + nxt, wn, wm, lane);
      load_act<T, 0>(fa, lds + nxt, wn, wm, lane);
      copy_stage(cur);
      load_unit<T>(ring[l1], w_rsrc, wbase, wc_u, (int)wgroup);
      mfma_part<T, 1, 0, T::TM, false>(acc, ring[u1], fb, sc);
      spread_vmem<T::TN * T::TM * T::MFMA_PER_UNIT, T::NCOPY + T::UNIT_LOADS>();
      pin_accumulators<T>(acc);
      __builtin_amdgcn_sched_barrier(0);
      advance_w();
      advance_a();
      sc = sn;
      select_scales<T>(sc, lane);
    } else {
      constexpr int u = SI % T::RING, l = (u + T::RING - 1) % T::RING;
      wait_vmcnt<T::WAIT_UNIT>();                  // unit u has landed
      __builtin_amdgcn_sched_barrier(0);
      mfma_part<T, 0, 0, T::TM / 2, ZERO>(acc, ring[u], fa, sc);
      pin_accumulators<T>(acc);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<T::WAIT_BARRIER, true>();         // stage g+1 has landed; reads of `cur` done
      barrier();
      __builtin_amdgcn_sched_barrier(0);
      load_act<T, 0>(fb, lds + nxt, wn, wm, lane);   // reads before the copies (see above)
      copy_stage(cur);
      load_unit<T>(ring[l], w_rsrc, wbase, wc_u, (int)wgroup);
      mfma_part<T, 0, T::TM / 2, T::TM, ZERO>(acc, ring[u], fa, sc);
      spread_vmem<T::TN * (T::TM - T::TM / 2), T::NCOPY + T::UNIT_LOADS>();
      pin_accumulators<T>(acc);
      __builtin_amdgcn_sched_barrier(0);
      advance_w();
      advance_a();
      fa = fb;
    }
    cur = nxt;
  };

  constexpr int SPG = T::STEPS_PER_GROUP;
  for (int i = 0; i < n_mine; ++i) {
    static_for<0, SPG>([&](auto si_c) __attribute__((always_inline)) {
      step(si_c, std::integral_constant<bool, decltype(si_c)::value == 0>{});
    });
    for (int gi = SPG; gi < nks; gi += SPG)
      static_for<0, SPG>([&](auto si_c) __attribute__((always_inline)) { step(si_c, std::false_type{}); });
    int n0, m0;
    tile_of(i, n0, m0);
    epilogue<T>(p, acc, n0 + wn * T::WN, m0 + wm * T::WM, lane, wn, wm, lds);
  }
  wait_vmcnt<0>();     // no copy into this workgroup's LDS may outlive it
}

// Tiles are dealt to one persistent workgroup per CU.
int cu_count() {
  static int count = 0;
  if (count == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      count = n;
    else
      count = 256;
  }
  return count;
}

// Environment switches, read once: DITQ_LOG=1 prints each GEMM launch's kernel and
// schedule to stderr; DITQ_FORCE_TILE=BMx256x128 (BM = 192 or 256) forces the token-tile
// height where the launcher chooses one (FP4 on the 2 x 2 grid), for experiments.
struct EnvFlags {
  bool log = false;
  int force_bm = 0;
  EnvFlags() {
    const char* l = std::getenv("DITQ_LOG");
    log = l != nullptr && l[0] == '1';
    if (const char* f = std::getenv("DITQ_FORCE_TILE")) {
      const int bm = std::atoi(f);
      if (bm == 192 || bm == 256) force_bm = bm;
      else std::fprintf(stderr, "ditq: DITQ_FORCE_TILE=%s ignored (token-tile height 192 or 256 expected)\n", f);
    }
  }
};
const EnvFlags& env_flags() {
  static const EnvFlags flags;
  return flags;
}

const char* fmt_name(int f) { return f == FMT_FP4 ? "FP4" : f == FMT_FP8 ? "FP8" : f == FMT_MX8 ? "MXFP8" : "NVFP4"; }
const char* epi_name(int e) {
  return e == EPI_IDENTITY ? "identity" : e == EPI_GATED_SILU ? "gated-SiLU" : e == EPI_QK_RMSNORM ? "QK-RMSNorm"
         : e == EPI_GELU_TANH ? "GELU-tanh" : "gated residual";
}

template <class T>
hipError_t launch(Params& p, hipStream_t stream) {
  p.tiles_m = (p.M + T::BM - 1) / T::BM;
  p.tiles_n = padded_rows(p.N) / T::BN;
  p.tiles = p.tiles_m * p.tiles_n;
  const int grid = p.tiles < cu_count() ? p.tiles : cu_count();
  if (env_flags().log)
    std::fprintf(stderr,
                 "ditq gemm: %s %s M=%d N=%d K=%d | tile 256x%d, %s grid, TM=%d, ring %d, LDS weight groups %d, "
                 "%d LDS stages of %d B | %d tiles on %d workgroups, %.3f rounds%s\n",
                 fmt_name(T::FMT), epi_name(T::EPI), p.M, p.N, p.K, T::BM, T::WAVES_N == 4 ? "4 x 1" : "2 x 2",
                 T::TM, T::RING, T::WLDS, T::STAGES, T::STAGE, p.tiles, grid, (double)p.tiles / grid,
                 p.out_f32 ? ", fp32 debug store" : "");
  if (p.out_f32 != nullptr)
    hipLaunchKernelGGL(gemm_kernel<typename T::Debug>, dim3(grid), dim3(T::NT), 0, stream, p);
  else
    hipLaunchKernelGGL(gemm_kernel<T>, dim3(grid), dim3(T::NT), 0, stream, p);
  return hipGetLastError();
}

// Token-tile height: on the 4 x 1 grid always 192 (TM = 6; at 256 tokens its 256
// accumulators leave too few registers, and the spilling kernel measured 5-8 %
// slower even where it saves a round of tiles: M = 2048 and 4096 with N = 16384).
// On the 2 x 2 grid 192 or 256 (TM = 3 or 4 per wave), whichever takes less time:
// rounds of tiles over the CUs times the time of one tile, a 256-token tile taking
// 1.35x a 192-token one (measured 1.34-1.37x: QK-RMSNorm head_dim 128, 4 against 3
// rounds, 100.1 against 102.9 us; head_dim 256, 5 against 3 rounds, 154.5 against
// 125.7 us; the gated residual, 3 against 2 rounds, 232.9 against 207.8 us).  FP8,
// MXFP8 and FP4 identity / gated-SiLU / GELU always take 192: with 256 their operand
// registers spill.  Weight ring: 8
// units on the FP4 4 x 1 grid when the k-steps come in groups of 4, else 4 (every 2 x 2
// grid, FP8 and MXFP8).
template <int FMT, int EPI, int HD = 0, int WLDS = wlds_for(FMT)>
hipError_t launch_cfg(Params& p, hipStream_t stream) {
  // 4 x 1 wave grid: 64 features x BM tokens per wave, every weight through registers.
  // Measured faster than the 2 x 2 grid with half its weight groups through LDS, for
  // FP4 (headline 122 vs 129 us) and FP8 (CFG-pair identity 316 vs 325 us): no weight
  // row is loaded by two waves, so the vector memory path carries less per k-step and
  // CU.  (FP4 with three fragment buffers takes the 2 x 2 grid again, below.)  MXFP8
  // and NVFP4 measured no faster and keep the 2 x 2 grid.  So does the gated residual, whose epilogue
  // spills on the 4 x 1 grid, and so does QK-RMSNorm: on the 4 x 1 grid a head spans
  // two or four waves (the epilogue handles it), but FP4 measured slower there
  // (head_dim 128: 109.6 vs 102 us; head_dim 256: 156 vs 127 us, where the 2 x 2
  // grid's 256-token tiles fit M = 4096 in 3 rounds) and FP8 no faster.
  constexpr bool grid41 = (FMT == FMT_FP4 || FMT == FMT_FP8) && EPI != EPI_QK_RMSNORM &&
                          EPI != EPI_GATE_RESIDUAL;
  if constexpr (FMT != FMT_FP4) {
    if constexpr (grid41) return launch<Tile<FMT, EPI, 6, 4, 0, HD, 4>>(p, stream);
    // NVFP4: every weight group in registers, like MXFP8 (same-box A/B against two
    // groups through LDS, outputs identical: gated-SiLU 347.2 -> 345.6 us, GELU
    // 297.3 -> 293.6, QK-RMSNorm head_dim 128 239.7 -> 238.6; no spills)
    else if constexpr (FMT == FMT_NV4) return launch<Tile<FMT, EPI, 3, 4, 0, HD>>(p, stream);
    else return launch<Tile<FMT, EPI, 3, 4, WLDS, HD>>(p, stream);
  } else {
    const int nks = p.K / 128;
    if constexpr (grid41) {
      // When the k-steps fill 6-step groups (K = 768, 1536, 3072, 12288, ...): the
      // 2 x 2 grid with every weight group in registers, a 4-unit ring and three
      // fragment buffers (192-token tiles, the gated residual's layout).  Each wave
      // reads half the tile's token rows from LDS (24 KB per k-step and CU against
      // the 4 x 1 grid's 48 KB), while the two waves of a row band both load its
      // weights (16 KB more per k-step and CU through the vector memory path).
      // Same-box A/B against the 4 x 1 grid's three-buffer kernel (itself 2-3 %
      // faster than that grid's two-buffer kernel), outputs identical, two boxes, 10
      // and 14 alternations: gated-SiLU 117.3 -> 115.3 and 118.1 -> 115.7 us, GELU
      // 112.1 -> 109.3 and 111.6 -> 108.7 us, identity 124.8 -> 122.6 us (identity
      // and GELU spill 4 VGPRs there).  Other K: the 4 x 1 grid, two buffers.
      if (nks % 6 == 0) return launch<Tile<FMT, EPI, 3, 4, 0, HD, 2, false, 3>>(p, stream);
      if (nks % 4 != 0) return launch<Tile<FMT, EPI, 6, 4, 0, HD, 4>>(p, stream);
      return launch<Tile<FMT, EPI, 6, 8, 0, HD, 4>>(p, stream);
    } else {
      const int cus = cu_count();
      const long tn = padded_rows(p.N) / 256;
      const long r3 = ((p.M + 191) / 192 * tn + cus - 1) / cus, r4 = ((p.M + 255) / 256 * tn + cus - 1) / cus;
      bool tm3 = r3 * 20 < r4 * 27;
      if (env_flags().force_bm) tm3 = env_flags().force_bm == 192;
      // 2 x 2 grid: a 4-unit weight ring (2 of the 4 groups come through LDS, so a
      // deeper ring only adds registers: with 8 units the QK-RMSNorm kernels spill
      // 3-24 VGPRs, and same-box A/B measured 4 units faster or level: QK-RMSNorm
      // head_dim 128 93.7 vs 96.9 us, 256 118.7 vs 119.9 us, the gated residual
      // 179.1 vs 179.9 us)
      // The gated residual (K = 12288 in the DiT MLP down projection) with every weight
      // group in registers and three fragment buffers when the k-steps fill 6-step
      // groups: same-box A/B 176.1 vs 181.7 us, outputs identical.  QK-RMSNorm
      // head_dim 128 with 192-token tiles: every weight group in registers with two
      // fragment buffers (three spill 8 VGPRs and measured slower, 97.9 us): each wave
      // reads only its half of the token rows from LDS; same-box A/B on two boxes,
      // outputs identical: 94.5 -> 91.9 and 85.8 -> 83.6 us.
      if constexpr (EPI == EPI_QK_RMSNORM && HD == 128) {
        if (tm3) return launch<Tile<FMT, EPI, 3, 4, 0, HD>>(p, stream);
      }
      if constexpr (EPI == EPI_GATE_RESIDUAL) {
        if (nks % 6 == 0) {
          if (tm3) return launch<Tile<FMT, EPI, 3, 4, 0, HD, 2, false, 3>>(p, stream);
          return launch<Tile<FMT, EPI, 4, 4, 0, HD, 2, false, 3>>(p, stream);
        }
      }
      if (tm3) return launch<Tile<FMT, EPI, 3, 4, WLDS, HD>>(p, stream);
      return launch<Tile<FMT, EPI, 4, 4, WLDS, HD>>(p, stream);
    }
  }
}

template <int FMT>
hipError_t launch_epi(Params& p, int epi, const RmsArgs* rms, hipStream_t stream) {
  switch (epi) {
    case EPI_IDENTITY:
      return launch_cfg<FMT, EPI_IDENTITY>(p, stream);
    case EPI_GATED_SILU:
      return launch_cfg<FMT, EPI_GATED_SILU>(p, stream);
    case EPI_GELU_TANH:
      return launch_cfg<FMT, EPI_GELU_TANH>(p, stream);
    case EPI_GATE_RESIDUAL:
      return launch_cfg<FMT, EPI_GATE_RESIDUAL>(p, stream);
    default:
      p.gamma_q = rms->gamma_q;
      p.gamma_k = rms->gamma_k;
      p.eps = rms->eps;
      p.n_heads = rms->n_heads;
      if (rms->head_dim == 128) return launch_cfg<FMT, EPI_QK_RMSNORM, 128>(p, stream);
      return launch_cfg<FMT, EPI_QK_RMSNORM, 256>(p, stream);
  }
}

}  // namespace

hipError_t launch_gemm(int fmt, const uint8_t* a_codes, const void* a_scales, const uint8_t* blob, int M, int N,
                       int K, int epi, const RmsArgs* rms, const ResidualArgs* gr, uint16_t* out, int ldo,
                       uint8_t* q_codes, uint8_t* q_scales, float* out_f32, hipStream_t stream) {
  const int Np = padded_rows(N);
  Params p{};
  p.a_codes = a_codes;
  p.a_scales = a_scales;
  p.w_codes = blob + kHeaderBytes;
  p.w_scales = blob + blob_scales_offset(fmt, Np, K);
  p.out = out;
  p.out_f32 = out_f32;
  p.q_codes = q_codes;
  p.q_scales = q_scales;
  p.M = M;
  p.N = N;
  p.K = K;
  p.ldo = ldo;
  p.a_bytes = (uint32_t)((size_t)M * (is_fp4_codes(fmt) ? K / 2 : K));
  p.w_bytes = (uint32_t)blob_code_bytes(fmt, Np, K);
  p.as_bytes = (uint32_t)((size_t)M * (fmt == FMT_FP8 ? 4 : fmt == FMT_NV4 ? K / 16 : K / 32));
  if (fmt == FMT_NV4) {
    p.a_tscale = reinterpret_cast<const float*>(static_cast<const uint8_t*>(a_scales) + nv4_act_tail(M, K) + 4);
    p.w_tscale = reinterpret_cast<const float*>(blob + kNvTensorScaleOff);
  }
  p.ws_bytes = (uint32_t)blob_scale_bytes(fmt, Np, K);
  if (gr) {
    p.residual = gr->residual;
    p.ldr = gr->ldr;
    p.gate = gr->gate;
    p.rows_per_gate = gr->rows_per_gate;
  }
  if (fmt == FMT_FP4) return launch_epi<FMT_FP4>(p, epi, rms, stream);
  if (fmt == FMT_NV4) return launch_epi<FMT_NV4>(p, epi, rms, stream);
  if (fmt == FMT_MX8) return launch_epi<FMT_MX8>(p, epi, rms, stream);
  return launch_epi<FMT_FP8>(p, epi, rms, stream);
}

}  // namespace ditq
