"""Pure-Python brute force for tiny cases (test infrastructure only).

An independent second route through the same step, used to pin the numpy
oracle: triple-loop matrix products and classical Gram-Schmidt applied twice
(CGS2) instead of LAPACK's Householder QR.  Gram-Schmidt produces the
positive-diagonal QR directly, because each diagonal entry is a norm.
Matrices are lists of rows of Python floats.
"""
from __future__ import annotations

import math
from typing import List

Mat = List[List[float]]


def zeros(m: int, n: int) -> Mat:
    return [[0.0] * n for _ in range(m)]


def transpose(a: Mat) -> Mat:
    return [list(col) for col in zip(*a)]


def matmul(a: Mat, b: Mat) -> Mat:
    m, k, n = len(a), len(b), len(b[0])
    assert all(len(row) == k for row in a)
    out = zeros(m, n)
    for i in range(m):
        for j in range(n):
            s = 0.0
            for p in range(k):
                s += a[i][p] * b[p][j]
            out[i][j] = s
    return out


def add(a: Mat, b: Mat, alpha: float = 1.0, beta: float = 1.0) -> Mat:
    return [[alpha * x + beta * y for x, y in zip(ra, rb)] for ra, rb in zip(a, b)]


def cgs2_qr(a: Mat):
    """Thin QR by classical Gram-Schmidt with one reorthogonalization.

    Returns (q, t) with a = q t, t upper triangular, t_jj = norm > 0.
    Raises ZeroDivisionError on an exactly dependent column.
    """
    m, n = len(a), len(a[0])
    cols = transpose(a)
    qcols: List[List[float]] = []
    t = zeros(n, n)
    for j in range(n):
        v = list(cols[j])
        for _ in range(2):
            coef = [sum(q[i] * v[i] for i in range(m)) for q in qcols]
            for p, q in enumerate(qcols):
                t[p][j] += coef[p]
                for i in range(m):
                    v[i] -= coef[p] * q[i]
        nrm = math.sqrt(sum(x * x for x in v))
        if nrm == 0.0:
            raise ZeroDivisionError("dependent column")
        t[j][j] = nrm
        qcols.append([x / nrm for x in v])
    return transpose(qcols), t


def colnorm(w: Mat) -> Mat:
    m, n = len(w), len(w[0])
    norms = [math.sqrt(sum(w[i][j] ** 2 for i in range(m))) for j in range(n)]
    return [[w[i][j] / norms[j] for j in range(n)] for i in range(m)]


def dion_step(X: Mat, G: Mat, R: Mat, V: Mat, eta: float, beta: float,
              variant: str):
    """The step by loops; returns (X', R', V', U, W)."""
    M = add(G, R)
    P = matmul(M, V)
    U, _ = cgs2_qr(P)
    W = matmul(transpose(M), U)
    if variant == "orth":
        Vb, _ = cgs2_qr(W)
    else:
        Vb = colnorm(W)
    X1 = add(X, matmul(U, transpose(Vb)), 1.0, -eta)
    R1 = [[beta * x for x in row] for row in add(M, matmul(U, transpose(W)), 1.0, -1.0)]
    return X1, R1, Vb, U, W
