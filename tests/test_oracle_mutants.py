"""The closed-form pins catch plausible mistakes.

Each mutant below is the oracle's step with one planted mistake (a dropped
term, a wrong operand, a transposed product, a sign, a missing sign fix).
Every mutant must disagree with at least one hand-derived closed form from
test_oracle_closed_forms, otherwise those pins would not pin anything.
"""
import numpy as np
import pytest

import oracle.dion_ref as ref
from oracle import DION, ORTH

from .test_oracle_closed_forms import _worked_3x2


def _qr_nosign(a):
    q, t = np.linalg.qr(np.asarray(a, dtype=np.float64), mode="reduced")
    return q, t


def _step(X, G, R, V, eta, beta, variant, mutate):
    qr = _qr_nosign if mutate == "no_sign_fix" else ref.qr_pos
    M = G if mutate == "drop_R" else G + R
    P = M @ V
    U, _ = qr(P)
    W = (M.T @ P) if mutate == "W_from_P" else (M.T @ U)
    if variant == ORTH:
        Vb, _ = qr(W)
    elif mutate == "rownorm":
        Vb = W / np.linalg.norm(W, axis=1, keepdims=True)
    else:
        Vb = ref.colnorm(W)
    Vx = V if mutate == "old_V_in_update" else Vb
    sign = 1.0 if mutate == "eta_sign" else -1.0
    X1 = X + sign * eta * (U @ Vx.T)
    Wr = Vb if mutate == "Vbar_in_residual" else W
    R1 = beta * (M - U @ Wr.T)
    if mutate == "no_beta":
        R1 = M - U @ Wr.T
    return X1, R1, Vb


def _worked_2x2_inputs():
    G = np.array([[2.0, 0.0], [4.0, 4.0]])
    R = np.eye(2)
    V = np.array([[1.0], [0.0]])
    X = np.array([[1.0, -1.0], [0.5, 2.0]])
    return X, G, R, V


def _closed_forms_hold(step):
    """True when a step function reproduces every hand-derived value."""
    ok = True
    # 2x2, r = 1 (see test_worked_2x2_rank1)
    X, G, R, V = _worked_2x2_inputs()
    s41 = np.sqrt(41.0)
    for variant in (DION, ORTH):
        X1, R1, V1 = step(X, G, R, V, 0.5, 0.25, variant)
        ok &= np.allclose(V1, np.array([[5.0], [4.0]]) / s41, atol=1e-12)
        ok &= np.allclose(X1, X - 0.5 / s41 * np.array([[3.0, 2.4], [4.0, 3.2]]),
                          atol=1e-12)
        ok &= np.allclose(R1, 0.25 * np.array([[0.0, -2.4], [0.0, 1.8]]), atol=1e-12)
    # 3x2, r = 2 (see test_worked_3x2_rank2)
    G, R, V, U, W, v_orth, v_dion, uv_orth, uv_dion = _worked_3x2()
    X = np.arange(6.0).reshape(3, 2) / 10.0
    for variant, vb, uv in ((ORTH, v_orth, uv_orth), (DION, v_dion, uv_dion)):
        X1, R1, V1 = step(X, G, R, V, 0.125, 0.75, variant)
        ok &= np.allclose(V1, vb, atol=1e-12)
        ok &= np.allclose(X1, X - 0.125 * uv, atol=1e-12)
        ok &= np.allclose(R1, 0.0, atol=1e-12)
    return bool(ok)


def test_unmutated_copy_passes():
    assert _closed_forms_hold(lambda *a: _step(*a, mutate=None))


@pytest.mark.parametrize("mutate", [
    "drop_R", "W_from_P", "rownorm", "old_V_in_update", "eta_sign",
    "Vbar_in_residual", "no_beta", "no_sign_fix",
])
def test_mutant_is_caught(mutate):
    assert not _closed_forms_hold(lambda *a: _step(*a, mutate=mutate))
