"""Pins of the float64 oracle against closed forms worked out by hand.

The pages print no numerical example of the step, so every expected value
here is derived by hand from the step's definition on the Orth-Dion page
(equation block and symbol list) and from textbook linear algebra; the
derivations are in the comments.  A dropped term (M = G instead of G + R),
a wrong operand (V_{t-1} instead of Vbar in the weight update, Vbar instead
of W in the residual), a transposed product or a sign error each change at
least one of these numbers.
"""
import math

import numpy as np
import pytest

from oracle import DION, ORTH, Breakdown, dion_step, qr_pos
from oracle.checks import orthonormality_error

S2 = math.sqrt(2.0)


def test_worked_2x2_rank1():
    # M = [[3,0],[4,5]] split as G + R with R = I.  V0 = e1.
    # P = M e1 = (3,4)^T, |P| = 5  ->  U = (0.6, 0.8)^T.
    # W = M^T U = (3*.6 + 4*.8, 5*.8) = (5, 4)^T, |W| = sqrt(41).
    # r = 1: both rules give Vbar = (5, 4)^T / sqrt(41).
    # X1 = X0 - eta U Vbar^T;  R1 = beta (M - U W^T) = beta [[0,-2.4],[0,1.8]].
    G = np.array([[2.0, 0.0], [4.0, 4.0]])
    R = np.eye(2)
    V = np.array([[1.0], [0.0]])
    X = np.array([[1.0, -1.0], [0.5, 2.0]])
    eta, beta = 0.5, 0.25
    s41 = math.sqrt(41.0)
    vbar = np.array([[5.0], [4.0]]) / s41
    u = np.array([[0.6], [0.8]])
    x1 = X - eta / s41 * np.array([[3.0, 2.4], [4.0, 3.2]])
    r1 = beta * np.array([[0.0, -2.4], [0.0, 1.8]])
    for variant in (DION, ORTH):
        res = dion_step(X, G, R, V, eta, beta, variant)
        np.testing.assert_allclose(res.U, u, atol=1e-15)
        np.testing.assert_allclose(res.W, [[5.0], [4.0]], atol=1e-14)
        np.testing.assert_allclose(res.V, vbar, atol=1e-15)
        np.testing.assert_allclose(res.X, x1, atol=1e-15)
        np.testing.assert_allclose(res.R, r1, atol=1e-15)


def _worked_3x2():
    # M = Q T with Q = [q1 q2], q1 = (2,2,1)/3, q2 = (-2,1,2)/3 (orthonormal)
    # and T = [[3,3],[0,3]]:  M = [[2,0],[2,3],[1,3]].  V0 = I (n = r = 2),
    # so P = M and U = Q (T has a positive diagonal).
    # W = M^T U = T^T Q^T Q = T^T = [[3,0],[3,3]].
    # Orth-Dion: QR of W: w1 = (3,3) -> v1 = (1,1)/sqrt2; w2 = (0,3) minus
    #   its projection 3/sqrt2 * v1 = (1.5,1.5) gives (-1.5,1.5) -> v2 =
    #   (-1,1)/sqrt2; diagonal (3 sqrt2, 3/sqrt2) > 0.
    # Dion: unit columns of W: (1,1)/sqrt2 and (0,1).
    # rank M = r, so R1 = beta (M - U T) = 0.
    M = np.array([[2.0, 0.0], [2.0, 3.0], [1.0, 3.0]])
    R = np.array([[1.0, 0.0], [0.0, 1.0], [0.0, 0.0]])
    G = M - R
    V = np.eye(2)
    U = np.array([[2.0, -2.0], [2.0, 1.0], [1.0, 2.0]]) / 3.0
    W = np.array([[3.0, 0.0], [3.0, 3.0]])
    v_orth = np.array([[1.0, -1.0], [1.0, 1.0]]) / S2
    v_dion = np.array([[1.0 / S2, 0.0], [1.0 / S2, 1.0]])
    # U Vbar^T worked row by row:
    uv_orth = np.array([[4.0 / (3 * S2), 0.0],
                        [1.0 / (3 * S2), 1.0 / S2],
                        [-1.0 / (3 * S2), 1.0 / S2]])
    uv_dion = np.array([[2.0 / (3 * S2), 2.0 / (3 * S2) - 2.0 / 3.0],
                        [2.0 / (3 * S2), 2.0 / (3 * S2) + 1.0 / 3.0],
                        [1.0 / (3 * S2), 1.0 / (3 * S2) + 2.0 / 3.0]])
    return G, R, V, U, W, v_orth, v_dion, uv_orth, uv_dion


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_worked_3x2_rank2(variant):
    G, R, V, U, W, v_orth, v_dion, uv_orth, uv_dion = _worked_3x2()
    X = np.arange(6.0).reshape(3, 2) / 10.0
    eta, beta = 0.125, 0.75
    res = dion_step(X, G, R, V, eta, beta, variant)
    np.testing.assert_allclose(res.U, U, atol=1e-15)
    np.testing.assert_allclose(res.W, W, atol=1e-14)
    vbar, uv = (v_orth, uv_orth) if variant == ORTH else (v_dion, uv_dion)
    np.testing.assert_allclose(res.V, vbar, atol=1e-15)
    np.testing.assert_allclose(res.X, X - eta * uv, atol=1e-15)
    np.testing.assert_allclose(res.R, np.zeros((3, 2)), atol=1e-14)


@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("m,n,r", [(7, 5, 2), (5, 7, 3), (6, 6, 6), (9, 4, 1)])
def test_diagonal_closed_form(variant, m, n, r):
    # M = rectangular diag(s1 > s2 > ...), V0 = [e1 .. er]:
    # P = M V0 = [s_j e_j], U = [e_j]; W = M^T U = [s_j e_j], Vbar = [e_j]
    # for both rules; X1 = X0 - eta sum_{j<r} e_j e_j^T;
    # R1 = beta diag(0, .., 0, s_{r+1}, ..).
    k = min(m, n)
    s = np.array([3.0 / (j + 1) for j in range(k)])
    M = np.zeros((m, n))
    M[np.arange(k), np.arange(k)] = s
    R = np.zeros((m, n))
    R[0, 0] = 0.5                      # arbitrary split of M into G + R
    G = M - R
    V = np.eye(n)[:, :r]
    X = np.full((m, n), 0.25)
    eta, beta = 0.01, 0.95
    res = dion_step(X, G, R, V, eta, beta, variant)
    E = np.zeros((m, n))
    E[np.arange(r), np.arange(r)] = 1.0
    np.testing.assert_allclose(res.U, np.eye(m)[:, :r], atol=1e-15)
    np.testing.assert_allclose(res.V, np.eye(n)[:, :r], atol=1e-15)
    np.testing.assert_allclose(res.X, X - eta * E, atol=1e-15)
    R1 = np.zeros((m, n))
    R1[np.arange(r, k), np.arange(r, k)] = beta * s[r:]
    np.testing.assert_allclose(res.R, R1, atol=1e-15)


def _planted(m, n, k, seed, sv=None):
    g = np.random.default_rng(seed)
    A, _ = np.linalg.qr(g.standard_normal((m, k)))
    B, _ = np.linalg.qr(g.standard_normal((n, k)))
    s = np.array(sv if sv is not None else [2.0 * 0.6 ** j for j in range(k)])
    return A, s, B, (A * s) @ B.T


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_exact_rank_r_recovery(variant):
    # rank M = r and span V0 = row(M): P = M V0 has full rank r with
    # col(P) = col(M), so U U^T M = M and R1 = 0.
    m, n, r = 12, 9, 3
    A, s, B, M = _planted(m, n, r, 5)
    Q, _ = np.linalg.qr(np.random.default_rng(6).standard_normal((r, r)))
    V = B @ Q
    G = 0.7 * M
    R = 0.3 * M
    res = dion_step(np.zeros((m, n)), G, R, V, 0.1, 0.9, variant)
    assert np.max(np.abs(res.R)) < 1e-14 * np.max(np.abs(M))


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_rank_below_r_completion(variant):
    # rank M = 2 < r = 4: orth(P) is undefined (breakdown) unless the
    # orthonormal completion is kept; then span U still contains col(M) and
    # the residual vanishes.
    m, n, r = 10, 8, 4
    _, _, B, M = _planted(m, n, 2, 7)
    V = np.linalg.qr(np.random.default_rng(8).standard_normal((n, r)))[0]
    with pytest.raises(Breakdown):
        dion_step(np.zeros((m, n)), M, np.zeros((m, n)), V, 0.1, 0.9, variant)
    if variant == DION:
        return   # colnorm of the completed W has no completion rule
    res = dion_step(np.zeros((m, n)), M, np.zeros((m, n)), V, 0.1, 0.9, variant,
                    on_rank_deficient="complete")
    assert orthonormality_error(res.U) < 1e-14
    assert np.max(np.abs(res.R)) < 1e-14


def test_zero_buffer_is_breakdown():
    # M = 0 (G = R = 0): P = 0 has no column space.
    m, n, r = 6, 5, 2
    V = np.eye(n)[:, :r]
    for variant in (ORTH, DION):
        with pytest.raises(Breakdown):
            dion_step(np.zeros((m, n)), np.zeros((m, n)), np.zeros((m, n)), V,
                      0.1, 0.9, variant)


def test_nonfinite_is_breakdown():
    m, n, r = 6, 5, 2
    G = np.ones((m, n)) + np.eye(m, n)
    G[2, 3] = np.nan
    with pytest.raises(Breakdown):
        dion_step(np.zeros((m, n)), G, np.zeros((m, n)), np.eye(n)[:, :r],
                  0.1, 0.9, ORTH)


def test_rank1_rules_coincide():
    # r = 1: the QR of one column is that column over its norm.
    g = np.random.default_rng(11)
    m, n = 9, 7
    X, G, R = (g.standard_normal((m, n)) for _ in range(3))
    V = g.standard_normal((n, 1))
    V /= np.linalg.norm(V)
    a = dion_step(X, G, R, V, 0.03, 0.9, ORTH)
    b = dion_step(X, G, R, V, 0.03, 0.9, DION)
    for f in ("X", "R", "V", "U"):
        np.testing.assert_allclose(getattr(a, f), getattr(b, f), atol=1e-14)


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_scale_invariance(variant):
    # (G, R) -> c (G, R): P, W scale by c, their QR / unit-column factors do
    # not, so X1 and V1 are unchanged and R1 scales by c.
    g = np.random.default_rng(12)
    m, n, r = 11, 8, 3
    X, G, R = (g.standard_normal((m, n)) for _ in range(3))
    V = np.linalg.qr(g.standard_normal((n, r)))[0]
    a = dion_step(X, G, R, V, 0.05, 0.8, variant)
    b = dion_step(X, 4.0 * G, 4.0 * R, V, 0.05, 0.8, variant)
    np.testing.assert_allclose(b.X, a.X, atol=1e-13)
    np.testing.assert_allclose(b.V, a.V, atol=1e-13)
    np.testing.assert_allclose(b.R, 4.0 * a.R, atol=1e-12)


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_orthogonal_equivariance(variant):
    # M -> Q1 M Q2^T, V -> Q2 V: U -> Q1 U (QR of Q1 P has the same
    # triangular factor), W -> Q2 W, Vbar -> Q2 Vbar (column norms and the
    # triangular factor of Q2 W are those of W), dX -> Q1 dX Q2^T,
    # R1 -> Q1 R1 Q2^T.
    g = np.random.default_rng(13)
    m, n, r = 10, 7, 3
    X, G, R = (g.standard_normal((m, n)) for _ in range(3))
    V = np.linalg.qr(g.standard_normal((n, r)))[0]
    Q1 = np.linalg.qr(g.standard_normal((m, m)))[0]
    Q2 = np.linalg.qr(g.standard_normal((n, n)))[0]
    a = dion_step(X, G, R, V, 0.05, 0.8, variant)
    b = dion_step(Q1 @ X @ Q2.T, Q1 @ G @ Q2.T, Q1 @ R @ Q2.T, Q2 @ V, 0.05,
                  0.8, variant)
    np.testing.assert_allclose(b.U, Q1 @ a.U, atol=1e-12)
    np.testing.assert_allclose(b.V, Q2 @ a.V, atol=1e-12)
    np.testing.assert_allclose(b.R, Q1 @ a.R @ Q2.T, atol=1e-12)
    np.testing.assert_allclose(b.X - Q1 @ X @ Q2.T, Q1 @ (a.X - X) @ Q2.T,
                               atol=1e-12)


@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_fixed_buffer_converges_to_top_singular_pairs(variant, beta):
    # Hold M fixed: beta = 0 with G = M*, or beta > 0 with G_t = M* - R_t.
    # Both rules then run orthogonal iteration (QR keeps the nested column
    # spans; column scaling does not change the QR of M Vbar), so U_t -> U_r
    # and Vbar_t -> V_r column by column with matching signs, and the
    # weight step U_t Vbar_t^T -> U_r V_r^T of numpy.linalg.svd.
    m, n, r = 14, 11, 3
    sv = [1.0 * 0.55 ** j for j in range(8)]
    _, _, _, Mstar = _planted(m, n, 8, 21, sv)
    Ufull, s, Vt = np.linalg.svd(Mstar)
    target = Ufull[:, :r] @ Vt[:r]
    V = np.linalg.qr(np.random.default_rng(22).standard_normal((n, r)))[0]
    X = np.zeros((m, n))
    R = np.zeros((m, n))
    eta = 1.0
    for _ in range(80):
        G = Mstar - R
        res = dion_step(X, G, R, V, eta, beta, variant)
        step = (X - res.X) / eta
        X, R, V = res.X, res.R, res.V
    np.testing.assert_allclose(step, target, atol=1e-10)
    np.testing.assert_allclose(R, beta * (Mstar - Ufull[:, :r] @ np.diag(s[:r]) @ Vt[:r]),
                               atol=1e-10)


def test_qr_pos_unique_factor():
    # For a full-rank input the positive-diagonal QR is unique: re-running on
    # a column-sign-flipped copy gives the same factor up to those signs.
    g = np.random.default_rng(30)
    A = g.standard_normal((12, 5))
    q, t = qr_pos(A)
    assert np.all(np.diag(t) > 0)
    np.testing.assert_allclose(q @ t, A, atol=1e-13)
    flips = np.array([1, -1, 1, -1, -1.0])
    q2, t2 = qr_pos(A * flips)
    np.testing.assert_allclose(q2, q * flips, atol=1e-13)
