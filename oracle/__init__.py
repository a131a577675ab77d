"""CPU oracle for the tiled-attention hot path.  TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never calls it, links it or falls back
to it; it shares no code with the HIP kernels (the only module both sides use
is the seeded input generator ``fa_inputs``, which holds no attention
arithmetic).

Two oracles:

* ``reference`` -- exact softmax attention and its gradients in float64,
  written from the plain definition.  FlashAttention is an exact algorithm
  (page 3, the section on FlashAttention's origins: tiling and kernel fusion
  reorganise the computation, they do not approximate it), and the repeated-
  maximum fix only changes the softmax shift (page 2, the section on where the
  bias comes from), to which softmax is invariant.  So both kernel variants
  target this one result.
* ``emulation`` -- the same tiled online-softmax recurrence, row by row, with
  the kernel's rounding sites (FP32 scores and running statistics, BF16 cast
  of the unnormalised probabilities before the PV product, BF16 output) and
  the repeated-maximum shift rule.  It exists to measure the rounding bias the
  pages describe, with the fix on and off; the parity gates use ``reference``.

``metrics`` holds the error statistics used by the tests and the benchmark.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
brute force, finite differences, library routines and invariants.  The one
part the pages give no number for -- the size of the tie bias and the shift
constants -- is "parity unpinned" (see ``emulation``).
"""
from . import reference, emulation, baseline, metrics  # noqa: F401
