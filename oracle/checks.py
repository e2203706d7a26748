"""Property checks on a step's outputs that hold at any size (test
infrastructure only).

They need only the inputs and outputs of a step, never the GPU path's
internals, and cost O((m + n) r^2) or a sampled subset of the m x n work, so
they apply where running the full float64 oracle would take too long.

All follow from the step as the Orth-Dion page defines it (equations 1-7 and
the symbol list): U has orthonormal columns; Vbar has orthonormal columns
(Orth-Dion) or unit columns (Dion); the weight change is -eta U Vbar^T; the
residual is beta times the part of M outside span(U).
"""
from __future__ import annotations

import numpy as np


def rel_fro(a, b) -> float:
    """||a - b||_F / ||b||_F (float64)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    num = np.linalg.norm(a - b)
    return float(num / den) if den > 0 else float(num)


def orthonormality_error(q) -> float:
    """max |q^T q - I|."""
    q = np.asarray(q, dtype=np.float64)
    return float(np.max(np.abs(q.T @ q - np.eye(q.shape[1]))))


def triangularity(q, a):
    """For the positive-diagonal thin QR a = q t: returns (lower, min_diag)
    where lower = max |(q^T a)_ij| over i > j relative to max |diag| and
    min_diag = min_j (q^T a)_jj / max |diag|.  A correct factor has lower
    ~ rounding and min_diag > 0."""
    q = np.asarray(q, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    t = q.T @ a
    d = np.diag(t)
    scale = np.max(np.abs(d))
    lower = np.max(np.abs(np.tril(t, -1))) if t.shape[0] > 1 else 0.0
    return float(lower / scale), float(np.min(d) / scale)


def left_factor_from_update(X0, X1, Vbar, eta):
    """Recover U from a step's outputs: X0 - X1 = eta U Vbar^T, so
    U = (X0 - X1) Vbar (Vbar^T Vbar)^{-1} / eta."""
    D = (np.asarray(X0, np.float64) - np.asarray(X1, np.float64)) / float(eta)
    Vb = np.asarray(Vbar, np.float64)
    gram = Vb.T @ Vb
    return np.linalg.solve(gram, (D @ Vb).T).T


def sampled_residual(M_rows, M_cols, U, rows, cols, beta):
    """R'[rows][:, cols] = beta (M - U W^T) restricted to the sample, with
    W[cols] = M[:, cols]^T U formed from full columns of M.

    M_rows: M[rows, :] (len(rows) x n); M_cols: M[:, cols] (m x len(cols)).
    """
    U = np.asarray(U, np.float64)
    Wc = np.asarray(M_cols, np.float64).T @ U              # len(cols) x r
    Mrc = np.asarray(M_rows, np.float64)[:, cols]
    return float(beta) * (Mrc - U[rows] @ Wc.T)
