"""CPU oracle for the mixed-precision training hot path.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously-correct
definition that the HIP kernels are checked against.  Only the test-suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product library (``mixed_precision_numerics_amd``) never
imports it and it never imports the product library; the two share no code.
The only module both sides use is ``synth`` (seeded input generators, which
hold none of the method's arithmetic).

Conventions
-----------
* Number formats are implemented from their bit layouts (sign / exponent /
  mantissa / bias) with exact float64 and integer arithmetic; no hardware or
  library low-precision conversion is used inside the oracle.
* An "FP32 operation" is evaluated exactly enough in float64 and then rounded
  once to FP32 with round-to-nearest-even.  For +, -, *, / and sqrt of FP32
  operands that equals the correctly rounded FP32 result (double rounding is
  innocuous because 53 >= 2*24 + 2; Figueroa, "When is double rounding
  innocuous?", SIGNUM Newsletter 1995).
* GEMM sums are in float64.

Modules
-------
formats   bit-exact codecs and rounding for FP32/FP16/BF16/E4M3/E5M2/E2M1
cast      scaled down-cast with amax capture
recipe    delayed-scaling amax history and scale update
scaler    dynamic loss scaler
adamw     unscale + overflow check + skip-or-apply AdamW on FP32 master
gemm      float64 GEMM reference, error bound, exact brute force
philox    Philox4x32-10 counter-based generator
hadamard  16-point random Hadamard transform
nvfp4     NVFP4 two-level quantizer (1x16 / 16x16 blocks, RNE / SR)
mlp       the tiny FP16 AMP training step (512->2048->GELU->10)
clip      FP32 gradient accumulation, global norm, clip coefficient
mx        MX block formats (UE8M0 scale per 32 elements)
blockwise fine-grained FP8 scaling (1x128 tiles, 128x128 blocks) and GEMM

Functions whose correctness cannot be pinned against anything outside the
oracle say "parity unpinned" in their docstring.
"""
