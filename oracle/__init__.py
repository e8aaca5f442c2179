"""CPU oracle for the SVDQuant W4A4 linear and the AWQ W4A16 GEMV.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
link this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library.

The oracle is a plain, slow, fp64-where-it-accumulates numpy restatement of
what the pages describe, step by step, in the pages' order:

* smoothing moves activation outliers into the weights, a small 16-bit
  low-rank branch takes the hardest part of the smoothed weight, the residual
  runs with 4-bit weights and 4-bit activations, and the two results are added
  (remio.ai page, section "SVDQuant moves hard values out of 4-bit";
  donmalab.com page, section on the core quantisation challenge);
* adaLN / modulation projections use 4-bit weights with 16-bit activations
  (AWQ W4A16; same pages, sections on the two layer types).

Numbers the pages leave open (group 64, ranks, fp16 scales, symmetric range,
alpha = 0.5, AWQ zero point) are fixed by the workload definition and listed,
with the reading taken, in the design notes.

Modules: ``numfmt`` (rounding to bf16/fp16), ``linalg`` (one-sided Jacobi SVD
and a randomised range finder), ``svdq`` (W4A4 path), ``awq`` (W4A16 path).

Pinned status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants, brute force on tiny inputs, library routines
or hand-derived fixtures under ``tests/golden/``. Image quality on trained
models is parity unpinned (no weights, prompts or calibration data exist here).
"""
