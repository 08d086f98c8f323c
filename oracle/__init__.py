"""Plain, slow, obviously-correct CPU oracle for the FP8 scaled linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``scaled_quantize_gemm_amd``) never imports it, and this package
never imports the product path: the two share no code.  The seeded input
generators both sides use live in ``workloads.py`` and contain none of the
method's arithmetic.

Sources (cited by page title and section):

* "Transformer Scaling" lesson reading (lab.mindcaptain.ai/reading/06):
  Concept deep dive 01 (E4M3 vs E5M2), Part 01 (scale and amax, delayed vs
  current scaling), Core vocabulary (amax, delayed scaling), Worked example
  01-02 (scale 448/240, 120 -> ~224, spike 300 clips at 448).
* "Week 14. Scaling laws, precision, parallelism" course page
  (snula.amonoc.com/course/en/week-14.html): the precision paragraph (bf16 has
  8 significant bits, 257 -> 256), the absmax paragraph (int8 worked example,
  per-tensor / per-block scales, MX 32-element scales, DeepSeek-V3 1x128 and
  128x128 blocks computed online), the FP8 bullet (E4M3 max 448, E5M2 max
  57,344, E4M3 for weights/activations and E5M2 for gradients) and the
  accumulation-precision bullet (64 + 3 = 64; 100 threes; promotion to fp32).
* Transformer Engine tutorial (juicytalk.now): the DelayedScaling recipe
  (HYBRID format, amax_history_len=16, amax_compute_algo="max"), the FP8
  metadata readback (scale, amax_history[0, :4]), the module tour
  (te.Linear(bias=True)) and the plain-PyTorch block (nn.GELU in the MLP).

Modules
-------
fp8        FP8 E4M3/E5M2 decode + saturating RNE encode, bf16 RNE, e8m0.
recipe     amax, delayed-scaling state and update, current-scaling scale rules.
quantize   per-tensor, 1x128, 128x128 and MX 1x32 quantizers; cast-transpose.
gemm       fp64 GEMM over dequantized operands plus the error-bound matrix.
epilogue   bias, exact GELU, SwiGLU over interleaved gate/up columns, FP8 output + amax.
layernorm  LayerNorm (biased variance, eps) followed by the quantizers.
absmax     int8 absmax example of the course page (a building-block check).
accum      FP8-rounded running sums (the accumulation-precision example).

Every function is pinned by ``tests/test_oracle_*.py`` to facts the pages print,
closed forms, invariants, library routines and brute force.  Readings taken
where the pages are silent are listed in each module's docstring.
"""

from . import fp8, recipe, quantize, gemm, epilogue, layernorm, absmax, accum  # noqa: F401
