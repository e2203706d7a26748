"""Oracle for the Dion / Orth-Dion optimizer step — TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 CPU implementation of the step as the Orth-Dion
documentation page writes it (its equation block: buffer, power-iteration
step, right factor, orthonormalized or column-normalized right factor, weight
update, residual, warm start).  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it.  The GPU library never calls it,
shares no code with it, and fails loudly when its own HIP build is missing.

Modules
  dion_ref    numpy float64 step (LAPACK Householder QR + sign fix)
  bruteforce  pure-Python loops (matmul, CGS2 Gram-Schmidt QR) for tiny cases
  checks      property checks that hold at any size (used by the tests)
"""
from .dion_ref import (  # noqa: F401
    DION, ORTH, Breakdown, StepResult, colnorm, dion_step, qr_pos, run_steps,
    step_diagnostics,
)
