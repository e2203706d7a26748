"""Pins of the oracle's multi-step driver, its diagnostics and the property
helpers of oracle/checks.py (CPU).

* run_steps is the step of the Orth-Dion page's equation block applied in
  turn (equation 7 carries V to the next step, equation 6 carries R): it
  equals an explicit loop of dion_step, and its float32-state mode equals
  that loop with X, R, V rounded to float32 after every step.  Independently
  of dion_step, with a fixed buffer (beta = 0, the same G every step) it
  runs orthogonal iteration, so the weight step converges to the top-r
  singular pairs of numpy.linalg.svd, in both modes.
* step_diagnostics reproduces the closed form of the diagonal case:
  P = diag(s_1 .. s_r), W = diag(s_1 .. s_r), gap s_r / s_{r+1}.
* checks.left_factor_from_update recovers U from X_t, X_{t+1} and Vbar, and
  checks.sampled_residual reproduces the oracle's R_{t+1} entry by entry.
"""
import numpy as np
import pytest

from oracle import DION, ORTH, dion_step, run_steps, step_diagnostics
from oracle.checks import left_factor_from_update, sampled_residual


def _state(m, n, r, seed):
    g = np.random.default_rng(seed)
    X = 0.02 * g.standard_normal((m, n))
    R = np.zeros((m, n))
    V = np.linalg.qr(g.standard_normal((n, r)))[0]
    grads = [g.standard_normal((m, n)) for _ in range(6)]
    return X, R, V, grads


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_run_steps_is_the_step_in_turn(variant):
    X, R, V, grads = _state(9, 7, 3, 1)
    x, r, v = X, R, V
    for G in grads:
        res = dion_step(x, G, r, v, 0.01, 0.95, variant)
        x, r, v = res.X, res.R, res.V
    out = run_steps(X, R, V, grads, 0.01, 0.95, variant)
    for a, b in zip(out, (x, r, v)):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_run_steps_float32_state(variant):
    X, R, V, grads = _state(9, 7, 3, 2)
    r32 = lambda a: a.astype(np.float32).astype(np.float64)
    x, r, v = X, R, V
    for G in grads:
        res = dion_step(x, G, r, v, 0.01, 0.95, variant)
        x, r, v = r32(res.X), r32(res.R), r32(res.V)
    out = run_steps(X, R, V, grads, 0.01, 0.95, variant, state_rounding="fp32")
    for a, b in zip(out, (x, r, v)):
        np.testing.assert_array_equal(a, b)
        assert np.array_equal(a, r32(a))          # every entry is a float32 value
    # rounding the state moves the trajectory, by about float32's rounding
    exact = run_steps(X, R, V, grads, 0.01, 0.95, variant)
    for a, b in zip(out, exact):
        d = np.linalg.norm(a - b) / np.linalg.norm(b)
        assert 0.0 < d < 1e-5
    with pytest.raises(ValueError):
        run_steps(X, R, V, grads, 0.01, 0.95, variant, state_rounding="fp16")


@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("rounding,tol", [(None, 1e-10), ("fp32", 1e-6)])
def test_run_steps_fixed_buffer_reaches_svd(variant, rounding, tol):
    # beta = 0 and the same G every step: M = G is fixed, the step is
    # orthogonal iteration, and U_t Vbar_t^T -> U_r V_r^T (numpy.linalg.svd)
    m, n, r = 13, 10, 3
    g = np.random.default_rng(3)
    A = np.linalg.qr(g.standard_normal((m, 8)))[0]
    B = np.linalg.qr(g.standard_normal((n, 8)))[0]
    M = (A * [1.0 * 0.5 ** j for j in range(8)]) @ B.T
    Uf, s, Vt = np.linalg.svd(M)
    target = Uf[:, :r] @ Vt[:r]
    V = np.linalg.qr(g.standard_normal((n, r)))[0]
    X0, R0 = np.zeros((m, n)), np.zeros((m, n))
    eta = 0.5
    x79, _, v79 = run_steps(X0, R0, V, [M] * 79, eta, 0.0, variant, state_rounding=rounding)
    x80, r80, _ = run_steps(x79, R0, v79, [M], eta, 0.0, variant, state_rounding=rounding)
    np.testing.assert_allclose((x79 - x80) / eta, target, atol=tol)
    np.testing.assert_array_equal(r80, np.zeros((m, n)))   # beta = 0


@pytest.mark.parametrize("m,n,r", [(7, 5, 2), (6, 9, 3), (5, 5, 5)])
def test_step_diagnostics_closed_form(m, n, r):
    k = min(m, n)
    s = np.array([4.0 / (j + 1) ** 2 for j in range(k)])
    M = np.zeros((m, n))
    M[np.arange(k), np.arange(k)] = s
    res = dion_step(np.zeros((m, n)), M, np.zeros((m, n)), np.eye(n)[:, :r], 0.01, 0.9, ORTH)
    d = step_diagnostics(res)
    assert d["cond_P"] == pytest.approx(s[0] / s[r - 1], rel=1e-12)
    assert d["cond_W"] == pytest.approx(s[0] / s[r - 1], rel=1e-12)
    if r < k:
        assert d["gap_r"] == pytest.approx(s[r - 1] / s[r], rel=1e-12)
    else:
        assert d["gap_r"] == float("inf")


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_left_factor_from_update(variant):
    X, R, V, grads = _state(11, 8, 4, 5)
    res = dion_step(X, grads[0], R, V, 0.03, 0.9, variant)
    U = left_factor_from_update(X, res.X, res.V, 0.03)
    np.testing.assert_allclose(U, res.U, atol=1e-12)


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_sampled_residual_matches_full_residual(variant):
    X, R, V, grads = _state(12, 9, 3, 6)
    R = 0.1 * np.random.default_rng(7).standard_normal(R.shape)
    res = dion_step(X, grads[1], R, V, 0.01, 0.9, variant)
    M = grads[1] + R
    rows, cols = np.array([0, 4, 11]), np.array([2, 3, 8])
    got = sampled_residual(M[rows], M[:, cols], res.U, rows, cols, 0.9)
    np.testing.assert_allclose(got, res.R[np.ix_(rows, cols)], atol=1e-13)
