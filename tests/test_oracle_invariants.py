"""Invariants of one step on random small inputs (oracle pins).

Each property follows from the step's definition on the Orth-Dion page
(equations 1-7, symbol list) and the Orth-Dion abstract's contrast between
the two right-factor rules:
  * U has orthonormal columns and U^T P is upper triangular with a positive
    diagonal (the unique positive-diagonal QR of P);
  * Orth-Dion: Vbar has orthonormal columns and Vbar^T W is upper triangular
    with positive diagonal; Dion: Vbar has unit columns, parallel to W's;
  * U^T R1 = 0, and R1 = beta (I - U U^T) M;
  * ||dX||_F = eta sqrt(r) for both rules; Orth-Dion's dX has all r nonzero
    singular values equal to eta (the dual-norm factor of one), Dion's has
    spectral norm between eta and eta sqrt(r).
"""
import math

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import DION, ORTH, dion_step
from oracle.checks import orthonormality_error, triangularity


@st.composite
def problems(draw):
    m = draw(st.integers(1, 24))
    n = draw(st.integers(1, 24))
    r = draw(st.integers(1, min(m, n)))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    variant = draw(st.sampled_from([DION, ORTH]))
    return m, n, r, seed, variant


def _inputs(m, n, r, seed):
    g = np.random.default_rng(seed)
    X = 0.02 * g.standard_normal((m, n))
    G = g.standard_normal((m, n))
    R = 0.5 * g.standard_normal((m, n))
    V = np.linalg.qr(g.standard_normal((n, r)))[0]
    return X, G, R, V


@settings(max_examples=150, deadline=None)
@given(problems())
def test_step_invariants(p):
    m, n, r, seed, variant = p
    X, G, R, V = _inputs(m, n, r, seed)
    eta, beta = 0.01, 0.95
    res = dion_step(X, G, R, V, eta, beta, variant)
    M = G + R
    # left factor
    assert orthonormality_error(res.U) < 1e-12
    low, dmin = triangularity(res.U, M @ V)
    assert low < 1e-12 and dmin > 0
    # right factor
    W = M.T @ res.U
    np.testing.assert_allclose(res.W, W, atol=1e-12)
    if variant == ORTH:
        assert orthonormality_error(res.V) < 1e-12
        low, dmin = triangularity(res.V, W)
        assert low < 1e-12 and dmin > 0
    else:
        np.testing.assert_allclose(np.linalg.norm(res.V, axis=0), 1.0, atol=1e-13)
        # parallel to W's columns, same direction
        cos = np.sum(res.V * W, axis=0) / np.linalg.norm(W, axis=0)
        np.testing.assert_allclose(cos, 1.0, atol=1e-12)
    # residual: beta times the part of M outside span(U)
    assert np.max(np.abs(res.U.T @ res.R)) < 1e-12 * max(1.0, np.max(np.abs(M)))
    proj = beta * (M - res.U @ (res.U.T @ M))
    np.testing.assert_allclose(res.R, proj, atol=1e-12)
    # weight change
    dX = X - res.X
    assert abs(np.linalg.norm(dX) - eta * math.sqrt(r)) < 1e-12
    sv = np.linalg.svd(dX, compute_uv=False)
    if variant == ORTH:
        np.testing.assert_allclose(sv[:r], eta, atol=1e-12)
    else:
        assert eta * (1 - 1e-12) <= sv[0] <= eta * math.sqrt(r) * (1 + 1e-12)
    assert np.all(sv[r:] < 1e-12)


@settings(max_examples=60, deadline=None)
@given(problems())
def test_residual_forms_agree(p):
    # Equation 6 prints U (U^T M); the GPU path reuses W^T = U^T M.
    m, n, r, seed, variant = p
    X, G, R, V = _inputs(m, n, r, seed)
    a = dion_step(X, G, R, V, 0.02, 0.9, variant, residual_form="reuse")
    b = dion_step(X, G, R, V, 0.02, 0.9, variant, residual_form="project")
    np.testing.assert_allclose(a.R, b.R, atol=1e-12)
