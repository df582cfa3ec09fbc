/*
 * ditq_measure.h -- C ABI of the measurement kernels that sit beside the fused
 * low-bit linear layer of ditq.h (same library, same general rules: device
 * pointers owned by the caller, no allocation or synchronisation, work enqueued
 * on `stream`, host-side argument checks before any HIP call, dit_status codes).
 *
 * They exist to measure the fused path against what it replaces and against the
 * hardware, not to compute it.
 */
#ifndef DITQ_MEASURE_H
#define DITQ_MEASURE_H

#include "ditq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Gated-SiLU as a separate pass over a bf16 GEMM output: the unfused form of
 * DIT_EPI_GATED_SILU.  Page "How fal made Ideogram V4 6x faster": paragraph 4
 * (the GEMM output is split in half and the halves multiplied after SiLU of the
 * first) and paragraph 3 (without fusion the output makes a full round trip to
 * HBM before the small op).
 *   out[m][j] = bf16(SiLU(c[m][j]) * c[m][j + N/2]),  0 <= j < N/2,
 *   SiLU(x) = x / (1 + e^-x), evaluated in fp32 with the hardware exp2 and
 *   reciprocal (the fused epilogue's arithmetic) and rounded to nearest even.
 * c_bf16: [M][ldc] bf16 bit patterns, columns [gate | up] in natural order (the
 * output of an identity GEMM with a DIT_EPI_IDENTITY blob); out_bf16: [M][ldo].
 * Each output element reads only its own row's two inputs.
 * Errors: DIT_EINVAL null pointer or M, N <= 0; DIT_EUNSUPPORTED N % 16 != 0;
 * DIT_EALIGN pointers not 16-byte aligned, ldc < N, ldo < N/2, or ldc / ldo not
 * multiples of 8; DIT_EDEVICE no gfx950 device or a launch error.  out must not
 * overlap c. */
dit_status dit_gated_silu_bf16(const void* c_bf16, int M, int N, int ldc, void* out_bf16, int ldo,
                               void* stream);

/* Debug form of the fused GEMM + epilogue: the same kernels as dit_gemm_epilogue and
 * dit_gemm_gate_residual (same arguments, formats, epilogues, shape rules and
 * errors), except that each output element is stored as the fp32 value the bf16
 * store would round, into out_f32 [M][ldo] (fp32, 16-byte aligned, ldo >= output
 * width, ldo % 4 == 0).  It shows the accuracy of the fused arithmetic before the
 * final bf16 rounding: the bf16 output of the other entry points equals the
 * round-to-nearest-even bf16 of this output, bit for bit.  Page "How fal made
 * Ideogram V4 6x faster", paragraphs 3-4 (the epilogues on the accumulator before
 * the one store).  gr must be non-NULL exactly when epi == DIT_EPI_GATE_RESIDUAL;
 * the residual must not overlap out_f32 (DIT_EINVAL). */
dit_status dit_gemm_epilogue_f32(dit_fmt fmt, const void* a_codes, const void* a_scales, const void* w_packed,
                                 int M, int N, int K, dit_epi epi, const dit_rmsnorm_params* rms,
                                 const dit_gate_residual_params* gr, float* out_f32, int ldo, void* stream);

/* Matrix-core throughput probe: `workgroups` workgroups of 4 waves, each wave
 * issuing iters x 8 independent v_mfma_scale_f32_32x32x64_f8f6f4 (FP4 E2M1
 * operands, unit scales) on register operands, with no memory traffic in its loop.
 * One launch performs workgroups * 4 * iters * 8 * 131072 FLOP.  out_u64 receives,
 * per workgroup w, out_u64[2w] = the s_memtime cycles wave 0 spent in its loop and
 * out_u64[2w + 1] = a checksum of its sums (its only purpose is to keep the work).
 * Timing the launch with events gives the sustained MFMA rate; cycles / time gives
 * the shader clock during it.
 * Errors: DIT_EINVAL null out_u64, workgroups outside [1, 65535] or iters outside
 * [1, 1 << 20]; DIT_EALIGN out_u64 not 8-byte aligned; DIT_EDEVICE as above. */
dit_status dit_mfma_fp4_probe(int workgroups, int iters, void* out_u64, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DITQ_MEASURE_H */
