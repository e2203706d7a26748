"""The numpy oracle against pure-Python loops on tiny inputs.

The brute-force route shares nothing with the oracle's numerical code: its
products are triple loops and its orth is classical Gram-Schmidt applied twice
(whose diagonal entries are norms, so positive by construction) rather than
LAPACK's Householder QR followed by a sign fix.
"""
import numpy as np
import pytest

from oracle import DION, ORTH, dion_step
from oracle import bruteforce as bf


def _tolist(a):
    return [list(map(float, row)) for row in np.asarray(a)]


@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("m,n,r,seed", [
    (1, 1, 1, 0), (1, 5, 1, 1), (6, 1, 1, 2), (4, 4, 4, 3), (12, 7, 3, 4),
    (7, 12, 5, 5), (12, 12, 6, 6), (9, 10, 9, 7), (3, 11, 2, 8),
])
def test_oracle_matches_bruteforce(variant, m, n, r, seed):
    g = np.random.default_rng(seed)
    X = 0.02 * g.standard_normal((m, n))
    G = g.standard_normal((m, n))
    R = 0.3 * g.standard_normal((m, n))
    V = np.linalg.qr(g.standard_normal((n, r)))[0]
    eta, beta = 0.01, 0.95
    ref = dion_step(X, G, R, V, eta, beta, variant)
    X1, R1, V1, U, W = bf.dion_step(_tolist(X), _tolist(G), _tolist(R),
                                    _tolist(V), eta, beta, variant)
    np.testing.assert_allclose(ref.U, np.array(U), atol=1e-12)
    np.testing.assert_allclose(ref.W, np.array(W), atol=1e-12)
    np.testing.assert_allclose(ref.V, np.array(V1), atol=1e-12)
    np.testing.assert_allclose(ref.X, np.array(X1), atol=1e-13)
    np.testing.assert_allclose(ref.R, np.array(R1), atol=1e-12)


def test_bruteforce_matmul_and_qr_basics():
    a = [[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]]
    b = [[1.0, 0.0, -1.0], [2.0, 1.0, 0.0]]
    assert bf.matmul(a, b) == [[5.0, 2.0, -1.0], [11.0, 4.0, -3.0], [17.0, 6.0, -5.0]]
    q, t = bf.cgs2_qr([[3.0, 1.0], [4.0, 2.0], [0.0, 2.0]])
    # first column (3,4,0)/5; t11 = 5; t12 = q1 . (1,2,2) = (3+8)/5
    assert abs(t[0][0] - 5.0) < 1e-15 and abs(t[0][1] - 11.0 / 5.0) < 1e-15
    assert abs(q[0][0] - 0.6) < 1e-15 and abs(q[1][0] - 0.8) < 1e-15
