"""CPU oracle for the fused low-bit DiT linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``bit_gemm_dit_amd``) never imports it and shares no code with it.

What it computes (plain, slow, obviously correct; float64 for floating point):

* ``formats``  -- decoding of bf16, FP4 E2M1, E8M0 and FP8 E4M3 codes.
* ``quant``    -- the on-the-fly activation quantizers and the weight quantizer:
  FP4 E2M1 with an E8M0 scale per 32-element K block, FP8 E4M3 with fp32
  per-row (activation) / per-column (weight) scales, MXFP8 (E4M3 with an
  E8M0 scale per 32-element K block) and NVFP4 (E2M1 with an E4M3 scale per
  16-element K block and an fp32 tensor scale).
* ``gemm``     -- decode codes and scales, multiply in float64.
* ``epilogue`` -- identity, gated-SiLU, per-head QK-RMSNorm, GELU (tanh form)
  and the gated residual update, in float64.
* ``packed``   -- decoder of the packed weight blob, written from the layout
  documented in ``include/ditq.h`` (used to check the packer bit-exactly).

The method is that of page "How fal made Ideogram V4 6x faster" (news.ditty.ir):
paragraph 2 (run the DiT in a 4-bit float format), paragraph 3 (epilogue fusion,
per-head RMSNorm, the head_dim 256 revisit schedule) and paragraph 4 (gated-SiLU
code snippet and the column interleave of B at packing time); FP8 as the second
path follows page "WaveSpeedAI X DataCrunch: FLUX real-time image inference on
B200" (engine list: BF16/FP8 mixed precision).

Parity pins: every function here is pinned by ``tests/test_oracle_*.py`` against
closed forms, exhaustive enumeration, exact-rational brute force and invariants.
The one part the pages cannot decide (which scale rule among the plausible
alternatives) is a documented convention; see ``quant.fp4_scale_byte``.
"""
