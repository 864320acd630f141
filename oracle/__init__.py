"""Plain CPU oracle for the block-quantized weight matvec y = W.x.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
helpers with the HIP library under ``block_quantized_weight_qgemv_amd/``, and
it imports nothing from it.

What it computes (dequantize, then an FP64 dot) is the plain definition of the
operation the pages describe:

* "Hand-Writing Gemma 4 Flash-Decoding + an FP4 Matvec Bonus (Part 2)",
  section "The assumption that failed the profiler": FP4-E2M1 weights with
  per-group scales, sign in bit 3 of the code, all eight magnitudes exact in
  BF16; an FP8 lm_head matvec with a per-row scale applied once; and section
  "The test that catches what parity misses": an FP64 host reference over the
  same bf16-rounded inputs.
* "perf(cuda/gemma4): decode is bound by 8-bit MLP weight bytes ... #683",
  section "Step 2 result": group-64 min-max affine 4/8-bit codes packed into
  u32 low-first, bf16 scales and biases rounded before q is computed.

Modules
  formats   bf16 / E2M1 / E4M3 closed-form decoders and round-to-nearest-even
            encoders.
  layout    unpackers (and packers) for nibble and u32 low-first code layouts.
  quantize  the offline quantizers (FP4 absmax, affine min-max, FP8 row absmax).
  gemv      dequantize-then-FP64-dot for each format, plus the conditioning
            mass A = sum |w x| used by the parity criterion.
  norm      RMSNorm of the activations rounded to bf16, the input of the
            fused norm-then-matvec variants (Part 2 post, "Where it landed").
  q8        the int8 activation route for affine 4-bit weights: activation
            blocks of 32 with an fp16 pair {d, s}, integer block dots and the
            bias applied through the block's activation sum ("perf(cuda):
            generalize Gemma 4 batched prefill ... dense Q4_K models",
            "Item C2").
  superblock  the two-level 4-bit super-block format (256-weight
            super-blocks with fp16 d and dmin, 32-weight sub-blocks with
            six-bit scale and min factors): its storage records, quantizer,
            exact dequantization, matvec and the pre-unpacked device
            layout (same issue, "Work Item C (C1) done", "Item C2", "All
            work items complete").

Every function is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_*``
against closed forms, library decoders, exact rational brute force or the
pages' own byte accounting.  Functions with no such pin say "parity unpinned".
"""

from . import formats, layout, quantize, gemv, norm, q8, superblock  # noqa: F401
