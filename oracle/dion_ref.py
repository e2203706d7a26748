"""Float64 oracle of one Dion / Orth-Dion step (test infrastructure only).

Source: the "Orth-Dion" documentation page (junaidaliop.github.io, zij/math/
orthdion), its equation block and the symbol list under it; the Dion rule
(column normalization of the right factor) is the replacement that page names
in its last sentence; the Orth-Dion abstract (thelatestinai.com, 2605.16341,
Abstract) explains it as scaling every column of the right factor to length
one.

Per call, with t the step index of the page:

  M    = G + R                      buffer (equation 1)
  P    = M V                        power-iteration step on the warm start
  U    = orth(P)                    (equation 2)
  W    = M^T U                      right factor (equation 3)
  Vbar = orth(W)          Orth-Dion (equation 4)
       = W diag(1/|w_j|)  Dion      (the page's replacement rule)
  X'   = X - eta U Vbar^T           (equation 5)
  R'   = beta (M - U W^T)           (equation 6; U^T M = W^T by equation 3)
  V'   = Vbar                       (equation 7: the warm start of step t+1)

orth(.) is the Q factor of a QR factorization, an orthonormal basis of the
column space (symbol list).  A thin QR is unique only up to column signs;
here the triangular factor is taken with a positive diagonal, which makes the
result unique for a full-rank input.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

DION = "dion"
ORTH = "orth"
_VARIANTS = (DION, ORTH)


class Breakdown(ArithmeticError):
    """The step is undefined: orth of a rank-deficient or non-finite factor,
    or a zero / non-finite column norm."""


def qr_pos(a: np.ndarray, on_rank_deficient: str = "raise",
           rel_tol: float = 1e-12):
    """Thin QR with positive diagonal: a = q @ t, q^T q = I, t upper
    triangular with t_jj > 0.

    Uses LAPACK Householder QR through numpy, then flips the sign of every
    column of q (and row of t) whose diagonal entry came out negative.

    on_rank_deficient:
      "raise"    raise Breakdown when |t_jj| <= rel_tol * max|t_jj| (or the
                 input is not finite);
      "complete" keep Householder's orthonormal completion for the deficient
                 columns (used only by tests of the exactly-low-rank case).
    """
    a = np.asarray(a, dtype=np.float64)
    if a.ndim != 2 or a.shape[0] < a.shape[1]:
        raise ValueError("qr_pos expects a tall (rows >= cols) matrix")
    if not np.all(np.isfinite(a)):
        raise Breakdown("non-finite input to orth")
    q, t = np.linalg.qr(a, mode="reduced")
    d = np.diag(t).copy()
    dmax = np.max(np.abs(d)) if d.size else 0.0
    deficient = (np.abs(d) <= rel_tol * dmax) | (dmax == 0.0)
    if deficient.any() and on_rank_deficient == "raise":
        raise Breakdown("orth of a rank-deficient matrix")
    s = np.where(d < 0.0, -1.0, 1.0)
    return q * s, t * s[:, None]


def colnorm(w: np.ndarray) -> np.ndarray:
    """Dion's right-factor rule: every column rescaled to unit Euclidean
    length.  No epsilon; a zero or non-finite norm is a breakdown."""
    w = np.asarray(w, dtype=np.float64)
    norms = np.sqrt(np.sum(w * w, axis=0))
    if not np.all(np.isfinite(norms)) or np.any(norms == 0.0):
        raise Breakdown("zero or non-finite column norm")
    return w / norms


@dataclasses.dataclass
class StepResult:
    X: np.ndarray      # X_{t+1}
    R: np.ndarray      # R_{t+1}
    V: np.ndarray      # V_t = Vbar_t (warm start of the next step)
    U: np.ndarray      # left factor U_t
    W: np.ndarray      # right factor W_t before normalization
    P: np.ndarray      # M_t V_{t-1}
    M: np.ndarray      # buffer M_t


def dion_step(X, G, R, V, eta, beta, variant: str,
              on_rank_deficient: str = "raise",
              residual_form: str = "reuse") -> StepResult:
    """One step on float64 copies of the inputs.

    X, G, R: m x n; V: n x r (r <= min(m, n)); eta, beta: scalars (pass the
    float32 value widened to float64 to mirror a float32 caller).

    residual_form: "reuse" forms U W^T (W^T = U^T M by equation 3), as the
    GPU path does; "project" forms U (U^T M) as equation 6 prints it.
    """
    if variant not in _VARIANTS:
        raise ValueError(f"variant must be one of {_VARIANTS}")
    X = np.asarray(X, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    m, n = X.shape
    if G.shape != (m, n) or R.shape != (m, n) or V.shape[0] != n:
        raise ValueError("shape mismatch")
    r = V.shape[1]
    if not 1 <= r <= min(m, n):
        raise ValueError("rank out of range")
    eta = float(eta)
    beta = float(beta)

    M = G + R                                         # equation 1
    P = M @ V                                         # equation 2, inner product
    U, _ = qr_pos(P, on_rank_deficient)               # equation 2, orth
    W = M.T @ U                                       # equation 3
    if variant == ORTH:
        Vbar, _ = qr_pos(W, on_rank_deficient)        # equation 4
    else:
        Vbar = colnorm(W)                             # Dion's rule
    X1 = X - eta * (U @ Vbar.T)                       # equation 5
    if residual_form == "reuse":
        R1 = beta * (M - U @ W.T)                     # equation 6
    else:
        R1 = beta * (M - U @ (U.T @ M))               # equation 6 as printed
    return StepResult(X=X1, R=R1, V=Vbar, U=U, W=W, P=P, M=M)


def _round32(a: np.ndarray) -> np.ndarray:
    return a.astype(np.float32).astype(np.float64)


def run_steps(X, R, V, grads, eta, beta, variant: str,
              state_rounding: Optional[str] = None):
    """Iterate the step over an iterable of gradients.

    state_rounding=None keeps the state in float64; "fp32" rounds X, R and V
    to float32 after every step (used to measure how far a float32-state
    trajectory drifts from the float64 one by rounding alone).
    Returns the final (X, R, V).
    """
    X = np.asarray(X, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    for G in grads:
        res = dion_step(X, G, R, V, eta, beta, variant)
        X, R, V = res.X, res.R, res.V
        if state_rounding == "fp32":
            X, R, V = _round32(X), _round32(R), _round32(V)
        elif state_rounding is not None:
            raise ValueError("state_rounding must be None or 'fp32'")
    return X, R, V


def step_diagnostics(res: StepResult) -> dict:
    """Conditioning of the two factors that orth sees, and the spectral gap
    of M at the rank (diagnostics only)."""
    def cond(a):
        s = np.linalg.svd(a, compute_uv=False)
        return float(s[0] / s[-1]) if s[-1] > 0 else float("inf")
    r = res.U.shape[1]
    sm = np.linalg.svd(res.M, compute_uv=False)
    gap = float(sm[r - 1] / sm[r]) if r < sm.size and sm[r] > 0 else float("inf")
    return {"cond_P": cond(res.P), "cond_W": cond(res.W), "gap_r": gap}
