/*
 * ditq.h -- C ABI of the fused low-bit linear layer for diffusion transformers
 * on AMD MI355X (gfx950).
 *
 * The layer: bf16 activations are quantized on the fly to a 4-bit float (FP4
 * E2M1, one E8M0 scale per 32 consecutive K elements), to FP8 E4M3 with one fp32
 * scale per row, to MXFP8 (E4M3, one E8M0 scale per 32 K elements), or to NVFP4
 * (E2M1, one E4M3 scale per 16 K elements and one fp32 scale per tensor); they are
 * multiplied with pre-packed low-bit weights on the
 * scaled MFMA units; the small op that follows the GEMM (identity, gated-SiLU,
 * per-head QK-RMSNorm) is applied to the fp32 accumulator before the single bf16
 * store.  Sources: page "How fal made Ideogram V4 6x faster" (news.ditty.ir),
 * paragraph 2 (4-bit float matmuls), paragraph 3 (epilogue fusion, per-head
 * RMSNorm, the head_dim 256 revisit schedule), paragraph 4 (gated-SiLU and the
 * packing-time column interleave of B); page "WaveSpeedAI X DataCrunch: FLUX
 * real-time image inference on B200", engine list (BF16/FP8 mixed precision).
 *
 * General rules for every entry point
 * -----------------------------------
 * - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *   allocates, frees or synchronises; each call only enqueues kernels on
 *   `stream` (a hipStream_t passed as void*, NULL = the default stream) and
 *   returns.  Asynchronous faults surface at the caller's next synchronisation.
 * - All argument checks run on the host before any HIP call, in this order:
 *     DIT_EINVAL       null pointer, M/N/K <= 0, unknown fmt/epi, missing or
 *                      inconsistent RMSNorm parameters
 *     DIT_EUNSUPPORTED a shape or combination the kernels do not implement
 *     DIT_EALIGN       a pointer not 16-byte aligned, or a leading dimension
 *                      smaller than the row width or not a multiple of 8 elements
 *     DIT_EDEVICE      no usable gfx950 device, or a launch error
 * - Outputs must not alias inputs.  Results are bitwise deterministic (no split-K,
 *   no atomics).  Calls
 *   on different streams may run concurrently.
 * - Matrices are row-major.  bf16 tensors are given as raw 16-bit patterns.
 */
#ifndef DITQ_H
#define DITQ_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DIT_OK = 0,
  DIT_EINVAL = 1,
  DIT_EUNSUPPORTED = 2,
  DIT_EALIGN = 3,
  DIT_EDEVICE = 4
} dit_status;

typedef enum {
  DIT_FMT_FP4_E2M1_MX32 = 1,   /* E2M1 codes + one E8M0 scale per 32 K elements */
  DIT_FMT_FP8_E4M3_ROWCOL = 2, /* OCP E4M3 codes + fp32 per-row / per-column scales */
  DIT_FMT_FP8_E4M3_MX32 = 3,   /* OCP E4M3 codes + one E8M0 scale per 32 K elements (MXFP8) */
  DIT_FMT_FP4_E2M1_NV16 = 4    /* E2M1 codes + one E4M3 scale per 16 K elements + fp32 tensor scale (NVFP4) */
} dit_fmt;

typedef enum {
  DIT_EPI_IDENTITY = 0,        /* out = bf16(C) */
  DIT_EPI_GATED_SILU = 1,      /* out[:, j] = bf16(SiLU(C[:, j]) * C[:, j + N/2]), j < N/2 */
  DIT_EPI_QK_RMSNORM = 2,      /* per-head RMSNorm on the Q and K heads of C = [Q | K | V] */
  DIT_EPI_GELU_TANH = 3,       /* out = bf16(0.5 C (1 + tanh(sqrt(2/pi) (C + 0.044715 C^3)))) */
  DIT_EPI_GATE_RESIDUAL = 4    /* out = bf16(residual + gate[sample] * C): dit_gemm_gate_residual */
} dit_epi;

/* Parameters of DIT_EPI_QK_RMSNORM (page "How fal made Ideogram V4 6x faster",
 * paragraph 3).  The GEMM output C has N = 3 * n_heads * head_dim columns laid
 * out [Q | K | V], each part head-major.  For every token row and every Q head h
 * (columns h*D .. h*D+D-1) and K head h (columns H*D + h*D ..):
 *     y[d] = x[d] / sqrt(mean_d(x^2) + eps) * gamma[d]
 * with gamma_q for the Q heads and gamma_k for the K heads (fp32 device
 * arrays of head_dim elements, shared by all heads).  V columns pass through.
 * head_dim 256 uses the two-half revisit schedule: the first 128 columns of a
 * head stay in registers with their partial sum of squares until the second
 * half's sum arrives, then both halves are normalised and stored. */
typedef struct {
  int head_dim;          /* 128 or 256 */
  int n_heads;           /* H, per Q / K / V */
  const float* gamma_q;  /* device, [head_dim] */
  const float* gamma_k;  /* device, [head_dim] */
  float eps;             /* > 0, e.g. 1e-6 */
} dit_rmsnorm_params;

/* Parameters of DIT_EPI_GATE_RESIDUAL, the residual update of adaLN-style DiT
 * blocks after the attention-output and MLP-down projections (the small op after
 * a big GEMM, fused so the result goes to HBM once: page "How fal made Ideogram
 * V4 6x faster", paragraphs 2-3):
 *     out[m][n] = bf16_RNE(residual[m][n] + gate[m / rows_per_gate][n] * C[m][n])
 * computed as one fp32 fused multiply-add; rows_per_gate tokens share a gate row
 * (one sample of a batch).  The residual may be the output itself (same pointer
 * and leading dimension) for an in-place update of the residual stream; any other
 * overlap of residual and output is DIT_EINVAL. */
typedef struct {
  const void* residual;  /* device, bf16 [M][ldr] */
  int ldr;               /* >= N, a multiple of 8 */
  const float* gate;     /* device, fp32 [ceil(M / rows_per_gate)][N] */
  int rows_per_gate;     /* > 0 */
} dit_gate_residual_params;

/* ---------------------------------------------------------------- size queries
 * Pure arithmetic, no device access; 0 means "unsupported arguments". */

/* Bytes of the packed weight blob written by dit_pack_weights.  Rows are padded
 * to Np = ceil(N / 256) * 256.  FP4: 256 + Np*K/2 + Np*K/32.  FP8: 256 + Np*K + 4*Np.
 * MXFP8: 256 + Np*K + Np*K/32.  NVFP4: 256 + Np*K/2 + Np*K/16. */
size_t dit_packed_weight_bytes(dit_fmt fmt, dit_epi epi, int N, int K);

/* Bytes of the activation codes / scales written by dit_quantize_act.
 * FP4: codes M*K/2, scales M*K/32.  FP8: codes M*K, scales 4*M.  MXFP8: codes M*K,
 * scales M*K/32.  NVFP4: codes M*K/2, scales M*K/16 + 16 + 2048. */
size_t dit_act_code_bytes(dit_fmt fmt, int M, int K);
size_t dit_act_scale_bytes(dit_fmt fmt, int M, int K);

/* ---------------------------------------------------------------- weight packer
 * The offline half of the layer: the weights are quantized once to the GEMM's
 * low-bit format and B's columns are permuted at packing time so that the
 * gate/up pairs of gated-SiLU sit next to each other (page "How fal made Ideogram
 * V4 6x faster", paragraph 2 for the 4-bit format, paragraph 4 for the
 * packing-time permutation of B).
 * Quantizes W (bf16 [N, K], row stride ldw elements; torch Linear layout, so
 * row n is output column n) and writes the packed blob (`packed`, at least
 * dit_packed_weight_bytes bytes, 256-byte aligned recommended).  Run once per
 * weight, offline.  `epi` selects the row order: DIT_EPI_GATED_SILU interleaves
 * the gate rows (0 .. N/2-1) with the up rows (N/2 .. N-1); the GEMM must then be
 * called with DIT_EPI_GATED_SILU too.  Blobs packed for every other epilogue are
 * identical (bar the epi field of the header) and interchangeable.
 *
 * Quantization rule, per weight row: FP4, MXFP8 and NVFP4 -- the same rule as
 * dit_quantize_act along K (NVFP4: with the tensor maximum of W); FP8 -- s_w[n] =
 * fl32(amax_n / 448) (1 if the row is zero), codes RNE_E4M3(fl32(w / s_w[n])).
 *
 * Blob layout (little-endian; the GEMM relies on it, tests decode it):
 *   header, 256 bytes: u32 magic 0x51544944 ("DITQ"), u32 layout version 2,
 *     u32 fmt, u32 epi, u32 N, u32 K, u32 Np, u32 0, u64 codes offset (256),
 *     u64 scales offset, u64 total bytes, then zeros.
 *   packed row p (0 <= p < Np) holds logical weight row perm(p): identity for
 *     IDENTITY / QK_RMSNORM; for GATED_SILU, with P = p / 64 and i = p % 64,
 *     perm(p) = 32P + i if i < 32 (gate) else N/2 + 32P + i - 32 (up), so a gate
 *     row and its up row land in the same lane of two adjacent 32-row groups of
 *     the MFMA output.  Rows p >= N are zero.
 *   FP4 codes: 1024-byte fragments (the B-operand registers of one
 *     32x32x64 MFMA); fragment (g, c), g < Np/32, c < K/64, at
 *     256 + (g*K/64 + c)*1024; its byte 16*L + b (lane L < 64, b < 16) holds
 *     the codes of packed row 32g + L%32 at k = 64c + 32*(L/32) + 2b (low
 *     nibble) and k + 1 (high nibble).
 *   FP4 scales: 128-byte records (s, g), s < K/128 (a 128-element K step),
 *     g < Np/32, at scales offset + (s*Np/32 + g)*128; byte 2*L + j is the E8M0
 *     scale of packed row 32g + L%32 for the 32-element K block 4s + 2j + L/32
 *     (the 16-bit word of lane L holds the scales of its two 64-K MFMA steps,
 *     picked with op_sel), so one K step of 256 packed rows is 1 KB contiguous.
 *   FP8 codes: 2048-byte fragments (g, c) at 256 + (g*K/64 + c)*2048; byte
 *     32*L + b holds the E4M3 code of packed row 32g + L%32 at
 *     k = 64c + 32*(b/16) + 16*(L/32) + b%16 (the 8-bit operand order of the
 *     32x32x64 MFMA: each lane holds two 16-element runs, and the 32-element
 *     block 64c + 32j is the j-th run of both lane groups).
 *   FP8 scales: fp32 [Np] at the scales offset, in packed row order.
 *   MXFP8 codes: the FP8 code layout.  MXFP8 scales: the FP4 scale layout (128-byte
 *     records (s, g), byte 2*L + j = the E8M0 scale of packed row 32g + L%32 for
 *     the K block 4s + 2j + L/32).
 *   NVFP4 codes: the FP4 code layout.  NVFP4 scales: 256-byte records (s, g) at
 *     scales offset + (s*Np/32 + g)*256; byte 4*L + 2*j + b is the E4M3 scale of
 *     packed row 32g + L%32 for the 16-element K block 8s + 4j + 2*(L/32) + b.  The
 *     fp32 tensor scale is stored in the header at byte 56 (byte 60 is work space
 *     of the packer).
 *
 * Supported: K % 128 == 0; N % 64 == 0 (GATED_SILU: N % 128 == 0); ldw >= K,
 * ldw % 8 == 0; w_bf16 and packed 16-byte aligned.  W must be finite. */
dit_status dit_pack_weights(dit_fmt fmt, dit_epi epi, const void* w_bf16, int N, int K,
                            int ldw, void* packed, void* stream);

/* ---------------------------------------------------------------- activation quantizer
 * Quantizes x (bf16 [M, K], row stride ldx elements) on the fly; a bit-exact
 * kernel (round to nearest, ties to even).
 *
 * FP4 (activation statistics change every diffusion iteration, so scales are
 * computed per call from the data -- page "Versnellende diffusiemodellen met
 * TheStage AI", section on acceleration and compression):
 *   per row and per 32-element K block: amax = max |x|;
 *   scale byte = clamp(floor(log2 amax) - 2 + 127, 0, 254), 0 if amax == 0;
 *   code = sign(x) | RNE_E2M1(min(|x| / 2^(byte-127), 6)), the sign bit copied
 *   from x even when the magnitude rounds to 0.
 *   Layout (K-panel-major, so that the GEMM copies a token tile of one K panel as
 *   one contiguous run): panel s = k / 128.  Codes: byte (s*M + m)*64 + (k%128)/2
 *   holds token m's codes at k (low nibble, k even) and k + 1 (high nibble).
 *   Scales: byte (s*M + m)*4 + (k%128)/32 is the E8M0 scale of token m's block
 *   k/32.  (Sizes M*K/2 and M*K/32 bytes.)
 * FP8:
 *   per row: s = fl32(amax / 448) (1 if the row is zero); code =
 *   RNE_E4M3(fl32(x / s)), both divisions IEEE fp32.  Codes K-panel-major with
 *   64-element panels: byte (s*M + m)*64 + k%64, s = k / 64, holds token m's code
 *   at k; scales fp32 [M].
 * MXFP8 (FP8 in the block-scaled structure of the FP4 path):
 *   per row and per 32-element K block: amax = max |x|;
 *   scale byte = clamp(floor(log2 amax) - 8 + 127, 0, 254), 0 if amax == 0 (the
 *   8 is the exponent of E4M3's largest magnitude, 448 = 1.75 * 2^8);
 *   code = RNE_E4M3(min(|x| / 2^(byte-127), 448)) with the sign of x.
 *   Codes in the FP8 layout (64-element panels); scales in the FP4 layout
 *   (byte (s*M + m)*4 + (k%128)/32, s = k / 128).
 * NVFP4 (the 4-bit format of page "How fal made Ideogram V4 6x faster", paragraph
 * 2, with its two levels of scaling), every step IEEE fp32:
 *   s_t = fl32(amax_tensor / 2688) (2688 = 6 * 448; 1 for an all-zero tensor);
 *   per row and 16-element K block: s_b = RNE_E4M3(min(fl32(amax_b / fl32(6 s_t)),
 *   448)); code = sign(x) | RNE_E2M1(min(|fl32(x / fl32(dec(s_b) s_t))|, 6)),
 *   magnitude 0 where s_b = 0.
 *   Codes in the FP4 layout.  Scales: byte (s*M + m)*8 + (k%128)/16, s = k / 128,
 *   then a 16-byte tail at byte M*K/16: u32 work space, then the fp32 tensor scale
 *   s_t, then 2048 bytes of work space (per-workgroup maxima).  Three kernel
 *   launches (the tensor maximum is a grid-wide reduction, in two launches); the
 *   scales buffer must be 16-byte aligned.
 *
 * Supported: K % 128 == 0, ldx >= K, ldx % 8 == 0, pointers 16-byte aligned
 * (FP4 and MXFP8 scales: any alignment).  x must be finite. */
dit_status dit_quantize_act(dit_fmt fmt, const void* x_bf16, int M, int K, int ldx,
                            void* codes, void* scales, void* stream);

/* ---------------------------------------------------------------- activation quantizer, no work space
 * For callers that cannot allocate or hand over work space: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same
 * quantization, codes and scales as dit_quantize_act, bit for bit, for every
 * format.  Only NVFP4 needs work space beyond its outputs (the tensor-maximum slot
 * and 512 per-workgroup maxima, 2052 bytes for any M and K): dit_quantize_act takes
 * it from the scale buffer's tail, this entry from a static array of the library
 * (one per device, held until the process ends), so its NVFP4 scale buffer needs
 * only M*K/16 + 16 bytes (the block scales, then the 16-byte tail whose fp32 tensor
 * scale at byte M*K/16 + 4 the GEMM reads).  Other formats: exactly
 * dit_quantize_act.  Allocates, frees and synchronises nothing.
 * NVFP4 calls on one device share the static work space, so calls that overlap on
 * one device (on different streams) race; calls on one stream are ordered.
 * Arguments, shapes (the same limits on M and K; larger sizes DIT_EUNSUPPORTED)
 * and errors as dit_quantize_act. */
dit_status dit_quantize_act_noalloc(dit_fmt fmt, const void* x_bf16, int M, int K, int ldx,
                                    void* codes, void* scales, void* stream);

/* ---------------------------------------------------------------- fused GEMM + epilogue, FP4
 * The big GEMM in the 4-bit format, C = A @ B (page "How fal made Ideogram V4 6x
 * faster", paragraph 4), with the small op that follows it applied to the fp32
 * accumulator before the one store, so the output makes a single trip to HBM
 * (same page, paragraphs 2-3: the matmuls in a 4-bit float format, epilogue
 * fusion of per-head RMSNorm and gated-SiLU).
 * out = epi(A W^T) with A the FP4 activations from dit_quantize_act (a_codes,
 * a_scales in its K-panel-major layout) and W the blob from dit_pack_weights
 * (FP4, packed for the same epi family).  The fp32 accumulator goes through the
 * epilogue and is stored once as bf16 (round to nearest even) into out_bf16
 * [M][ldo]; the output width is N/2 for GATED_SILU and N otherwise.
 * `rms` must be non-NULL exactly when epi == DIT_EPI_QK_RMSNORM (host pointer to
 * the struct; the gammas inside are device pointers), with
 * N == 3 * n_heads * head_dim and head_dim in {128, 256}.  DIT_EPI_GATE_RESIDUAL
 * needs its parameters, which dit_gemm_gate_residual takes (here: DIT_EINVAL).
 * Supported: M >= 1 (any), K % 128 == 0, N % 64 == 0 (GATED_SILU: N % 128 == 0),
 * ldo >= output width, ldo % 8 == 0, pointers 16-byte aligned. */
dit_status dit_gemm_q4_epilogue(const void* a_codes, const void* a_scales, const void* w_packed,
                                int M, int N, int K, dit_epi epi, const dit_rmsnorm_params* rms,
                                void* out_bf16, int ldo, void* stream);

/* ---------------------------------------------------------------- fused GEMM + epilogue + FP4 output
 * The FP4 GEMM of dit_gemm_q4_epilogue whose epilogue also quantizes its output
 * for the next GEMM, so the output need not be read back by a separate
 * dit_quantize_act pass: the small op after each big GEMM is fused so that its
 * result goes to HBM once, and activations are quantized on the fly (page "How
 * fal made Ideogram V4 6x faster", paragraphs 2-3).
 *   y = bf16_RNE(epi(A W^T)) -- the value dit_gemm_q4_epilogue stores --
 *   (out_codes, out_scales) = FP4 quantization of y exactly as dit_quantize_act
 *   computes it (same block rule, rounding and K-panel-major layout), for M rows
 *   and K' = output width (N/2 for GATED_SILU, N otherwise) columns; sizes
 *   dit_act_code_bytes(FP4, M, K') and dit_act_scale_bytes(FP4, M, K').
 * out_bf16 may be NULL (then only the quantized output is written and ldo is
 * ignored); otherwise it is written as by dit_gemm_q4_epilogue.  The quantized
 * output equals dit_quantize_act applied to that bf16 output, bit for bit.
 * Supported: as dit_gemm_q4_epilogue, plus K' % 256 == 0; out_codes and
 * out_scales 16-byte aligned and not aliasing any input. */
dit_status dit_gemm_q4_epilogue_q4(const void* a_codes, const void* a_scales, const void* w_packed,
                                   int M, int N, int K, dit_epi epi, const dit_rmsnorm_params* rms,
                                   void* out_bf16, int ldo, void* out_codes, void* out_scales,
                                   void* stream);

/* ---------------------------------------------------------------- fused GEMM + epilogue, FP8
 * The same fused GEMM in FP8 E4M3, the second precision beside the 4-bit path
 * (page "WaveSpeedAI X DataCrunch: FLUX real-time image inference on B200",
 * engine list: BF16/FP8 mixed precision; the epilogues as on page "How fal made
 * Ideogram V4 6x faster", paragraphs 3-4).
 * out = epi((A W^T) * s_a[m] * s_w[n]) with A the E4M3 codes (K-panel-major) and
 * fp32 row scales [M] from dit_quantize_act, W an FP8 blob.  epi is IDENTITY,
 * GATED_SILU or GELU_TANH (QK_RMSNORM and GATE_RESIDUAL, which need parameters,
 * return DIT_EUNSUPPORTED here; dit_gemm_epilogue and dit_gemm_gate_residual take
 * them).  Same shape rules as the FP4 entry point
 * (a_scales 4-byte aligned). */
dit_status dit_gemm_q8_epilogue(const void* a_codes, const float* a_scales, const void* w_packed,
                                int M, int N, int K, dit_epi epi,
                                void* out_bf16, int ldo, void* stream);

/* ---------------------------------------------------------------- fused GEMM + epilogue, any format
 * The GEMM + epilogue of the entry points above for every format and epilogue:
 *   fmt = DIT_FMT_FP4_E2M1_MX32: exactly dit_gemm_q4_epilogue;
 *   fmt = DIT_FMT_FP8_E4M3_ROWCOL: dit_gemm_q8_epilogue (a_scales: fp32 [M]),
 *     plus QK_RMSNORM, applied to (A W^T) * s_a[m] * s_w[n];
 *   fmt = DIT_FMT_FP8_E4M3_MX32: out = epi(A W^T), A and W MXFP8 (E4M3 codes with
 *     E8M0 block scales applied inside the product, as for FP4), every epilogue;
 *   fmt = DIT_FMT_FP4_E2M1_NV16: out = epi((sum_k A W) * s_t(A) * s_t(W)) with the
 *     E4M3 block scales inside the sum: the NVFP4 product, exact up to fp32
 *     accumulation (the elements and block scales are multiplied exactly in
 *     f16 before an f16 matrix multiply), every epilogue.
 * FP8 as the safer precision beside the 4-bit format: page "WaveSpeedAI X
 * DataCrunch: FLUX real-time image inference on B200", engine list; page on
 * FLUX.1-dev inference optimization with LoRA (aitime.ge), FP8 quantization as
 * the best speed / memory trade-off.  The epilogues: page "How fal made Ideogram
 * V4 6x faster", paragraphs 3-4.
 * A and W must come from dit_quantize_act / dit_pack_weights with the same fmt
 * (W packed for the same epi family).  Arguments, shapes, alignment and error
 * codes as dit_gemm_q4_epilogue (FP8 row scales: 4-byte aligned). */
dit_status dit_gemm_epilogue(dit_fmt fmt, const void* a_codes, const void* a_scales, const void* w_packed,
                             int M, int N, int K, dit_epi epi, const dit_rmsnorm_params* rms,
                             void* out_bf16, int ldo, void* stream);

/* ---------------------------------------------------------------- fused GEMM + gated residual
 * out = bf16(residual + gate[m / rows_per_gate] * C) with C = A W^T in any format
 * (FP8 row/column: C includes s_a[m] * s_w[n]), the DIT_EPI_GATE_RESIDUAL
 * epilogue (parameters above).  Width N, weights packed for any epi but
 * GATED_SILU.  Arguments, shapes and errors as dit_gemm_epilogue; residual and
 * gate 16-byte aligned, ldr >= N and ldr % 8 == 0 (else DIT_EALIGN); gr NULL or a
 * NULL member, rows_per_gate <= 0, or a partial overlap of residual and output:
 * DIT_EINVAL. */
dit_status dit_gemm_gate_residual(dit_fmt fmt, const void* a_codes, const void* a_scales, const void* w_packed,
                                  int M, int N, int K, const dit_gate_residual_params* gr,
                                  void* out_bf16, int ldo, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* dit_status_str(dit_status status);

/* Detail of the most recent DIT_EDEVICE returned on the calling thread (the
 * failing HIP call and its error string); "" if there was none.  The pointer
 * stays valid until the thread's next failing call. */
const char* dit_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DITQ_H */
