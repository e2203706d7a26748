"""The step's invariants, checked on libdion's own outputs (GPU).

Independent of the oracle: the properties the Dion and Orth-Dion pages
give the update, at float32 tolerances, on shapes that cross tile
boundaries.
* V̄ᵀV̄ = I (Orth-Dion) or unit columns of V̄ (Dion).
* ‖ΔX‖_F = η √r for both variants (U has orthonormal columns; V̄ has
  orthonormal or unit columns).
* Orth-Dion: every nonzero singular value of ΔX is η (the dual-norm factor
  is one).  Dion: η ≤ ‖ΔX‖₂ ≤ η √r.
* Uᵀ R_new = 0: the new residual has no component in span(U).  U is
  recovered from the outputs as U = −ΔX V̄ (V̄ᵀV̄)⁻¹ / η (the oracle's
  checks.left_factor_from_update).
"""
import math

import numpy as np
import pytest

from oracle import DION, ORTH
from oracle.checks import left_factor_from_update
from workloads.configs import MatrixSpec, Workload

from .gpuhelp import Case, f32, say

pytestmark = pytest.mark.gpu

SHAPES = [(300, 200, 40), (257, 129, 17), (512, 384, 128), (700, 300, 250)]


def _wl(m, n, r, seed):
    return Workload(name=f"inv{m}x{n}r{r}", seed=seed, mats=(MatrixSpec(0, "W", 0, m, n, r),),
                    g_dtype="bf16", g_kind="planted", noise=(0.05,), planted_rank=min(m, n) // 2,
                    eta=0.01, beta=0.95, steps=1, variants=("orth", "dion"))


@pytest.mark.parametrize("m,n,r", SHAPES)
@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_update_invariants(gpu_lib, m, n, r, variant, arith):
    wl = _wl(m, n, r, seed=7 + m)
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    say(f"invariants {m}x{n} r={r} {variant} {arith}")
    x0 = c.X.double().cpu().numpy()
    gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, variant, math=arith)
    eta = float(f32(wl.eta))
    dx = c.X.double().cpu().numpy() - x0
    vb = c.V.double().cpu().numpy()
    r_new = c.R.double().cpu().numpy()

    gram = vb.T @ vb
    if variant == ORTH:
        assert np.abs(gram - np.eye(r)).max() < 1e-5
    else:
        assert np.abs(np.diag(gram) - 1.0).max() < 1e-5

    assert abs(np.linalg.norm(dx) - eta * math.sqrt(r)) < 1e-4 * eta * math.sqrt(r)

    sv = np.linalg.svd(dx, compute_uv=False)
    assert sv[r:].max(initial=0.0) < 1e-4 * eta   # rank r
    if variant == ORTH:
        assert np.abs(sv[:r] - eta).max() < 1e-4 * eta
    else:
        assert eta * (1 - 1e-4) <= sv[0] <= eta * math.sqrt(r) * (1 + 1e-4)

    u = left_factor_from_update(x0, x0 + dx, vb, eta)
    assert np.abs(u.T @ u - np.eye(r)).max() < 1e-4
    # residual orthogonal to span(U), relative to the residual's own size
    assert np.linalg.norm(u.T @ r_new) < 1e-4 * np.linalg.norm(r_new)
