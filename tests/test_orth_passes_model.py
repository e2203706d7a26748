"""A numpy model of libdion's orth() over the whole range of conditioning
(CPU): the decision between one CholeskyQR pass, CholeskyQR2 and the
shifted first pass, and the arithmetic of each part, restated so that the
design's claims can be checked without a GPU.

The model follows the library's roles, not its kernels:
* first pass: a float64 Gram matrix with the sliced Gram's error (each
  entry off by up to 2^-30 max|q_i| max|q_j| per row, added like independent
  roundings), a float64 Cholesky factorization S = T^T T, and Q T^{-1} in
  float32;
* the decision uses t = trace(C^{-1}) for the column-scaled Gram matrix C
  (t = sum_ij S_ii (T^{-1})_ij^2, between 1/lambda_min(C) and r/lambda_min(C)):
  one pass while t <= 1e3 r and every pivot ratio d_j / S_jj >= 1e-6; the
  shifted first pass when t > 1e7 r, a pivot ratio is below 1e-8 or a pivot
  fails; a second pass otherwise;
* the shifted pass factors S + s diag(S) of the exact float64 Gram matrix,
  s = max((r rows + r^2) 2^-50, 2^-30);
* two-pass matrices take both triangular multiplies in float64, rounded
  once to float32; the second pass breaks down below a pivot ratio of
  r 2^-40.

Claims checked: the result matches the oracle's Householder Q factor of the
same float32 factor to float32 accuracy from kappa = 1e2 to 1e7; each kappa
takes the path the thresholds give; exactly dependent and zero columns are
breakdowns, as the oracle's are.  The GPU kernels are checked against the
oracle in test_gpu_orth_range.py."""
import numpy as np
import pytest

from oracle import Breakdown, qr_pos

RATIO_TWO, RATIO_RETRY = 1e-6, 1e-8
TRACE_TWO, TRACE_RETRY = 1e3, 1e7


class ModelBreakdown(Exception):
    pass


def _chol_ratios(S, tol):
    """float64 Cholesky S = T^T T with the library's pivot test (pivot >
    tol * S_jj, finite); returns (T, ratios) or raises ModelBreakdown at the
    first failed pivot."""
    r = S.shape[0]
    A = S.copy()
    T = np.zeros_like(S)
    ratios = np.empty(r)
    d = np.diag(S).copy()
    for j in range(r):
        piv = A[j, j]
        if not (piv > tol * d[j] and np.isfinite(piv)):
            raise ModelBreakdown(j)
        ratios[j] = piv / d[j]
        T[j, j] = np.sqrt(piv)
        T[j, j + 1:] = A[j, j + 1:] / T[j, j]
        A[j + 1:, j + 1:] -= np.outer(T[j, j + 1:], T[j, j + 1:])
    return T, ratios


def _sliced_gram(Q32, rng):
    Q = Q32.astype(np.float64)
    S = Q.T @ Q
    mx = np.abs(Q).max(axis=0)
    rows = Q.shape[0]
    E = rng.standard_normal(S.shape) * np.sqrt(rows) * 2.0 ** -30 * np.outer(mx, mx)
    return S + (E + E.T) / 2


def shift_of(rows, r):
    return max((r * rows + r * r) * 2.0 ** -50, 2.0 ** -30)


def model_orth(Q32, seed=0):
    """Returns (result float32, path) with path in {"one", "two", "retry"}."""
    rng = np.random.default_rng(seed)
    rows, r = Q32.shape
    S = _sliced_gram(Q32, rng)
    try:
        T, ratios = _chol_ratios(S, RATIO_RETRY)
        Ti = np.linalg.inv(T)
        trace = np.sum(np.diag(S)[:, None] * Ti ** 2)
        if not trace <= TRACE_RETRY * r:
            path = "retry"
        elif trace > TRACE_TWO * r or ratios.min() < RATIO_TWO:
            path = "two"
        else:
            path = "one"
    except ModelBreakdown:
        path = "retry"
    if path == "one":
        return (Q32 @ Ti.astype(np.float32)).astype(np.float32), path
    if path == "retry":
        S64 = Q32.astype(np.float64).T @ Q32.astype(np.float64)
        s = shift_of(rows, r)
        A = S64 + np.diag(s * np.diag(S64))
        try:
            T, _ = _chol_ratios(A, 0.5 * s)
        except ModelBreakdown:
            raise Breakdown("shifted factorization")
    Q1 = (Q32.astype(np.float64) @ np.linalg.inv(T)).astype(np.float32)
    S2 = Q1.astype(np.float64).T @ Q1.astype(np.float64)
    try:
        T2, _ = _chol_ratios(S2, r * 2.0 ** -40)
    except ModelBreakdown:
        raise Breakdown("second pass")
    return (Q1.astype(np.float64) @ np.linalg.inv(T2)).astype(np.float32), path


def planted_factor(rows, r, kappa, seed):
    """rows x r float32 factor with nearly collinear columns: a random mix
    of r orthonormal directions weighted by a spectrum from 1 to 1/kappa."""
    g = np.random.default_rng(seed)
    A, _ = np.linalg.qr(g.standard_normal((rows, r)))
    Z, _ = np.linalg.qr(g.standard_normal((r, r)))
    s = np.logspace(0, -np.log10(kappa), r)
    return ((A * s) @ Z).astype(np.float32)


@pytest.mark.parametrize("kappa,path", [(1e2, "one"), (1e3, "two"), (1e4, "two"),
                                        (1e6, "retry"), (1e7, "retry")])
@pytest.mark.parametrize("rows,r", [(256, 16), (700, 96)])
def test_model_matches_householder_over_the_range(kappa, path, rows, r):
    Q = planted_factor(rows, r, kappa, seed=rows + r)
    sv = np.linalg.svd(Q.astype(np.float64), compute_uv=False)
    assert sv[0] / sv[-1] == pytest.approx(kappa, rel=0.5)
    U, taken = model_orth(Q)
    assert taken == path, (kappa, taken)
    ref, _ = qr_pos(Q.astype(np.float64))
    err = np.linalg.norm(U - ref) / np.linalg.norm(ref)
    orth = np.abs(U.astype(np.float64).T @ U - np.eye(r)).max()
    assert err < 2e-6, (kappa, taken, err)
    assert orth < 2e-6, (kappa, taken, orth)


def test_model_duplicate_columns_break_down():
    Q = planted_factor(256, 16, 10.0, seed=3)
    Q[:, 7] = Q[:, 6]
    with pytest.raises(Breakdown):
        model_orth(Q)
    with pytest.raises(Breakdown):
        qr_pos(Q.astype(np.float64))


def test_model_zero_column_breaks_down():
    Q = planted_factor(256, 16, 10.0, seed=4)
    Q[:, 3] = 0.0
    with pytest.raises(Breakdown):
        model_orth(Q)
