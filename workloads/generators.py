"""Seeded, randomly addressable input streams.

Every random draw comes from ``numpy.random.default_rng([seed, i, s])``
(PCG64 seeded by the sequence), with ``seed`` the workload number, ``i`` the
matrix index in the stack and ``s`` the stream: ``s = 0`` is the init stream,
``s = t + 1`` feeds step ``t``.  Any matrix at any step can therefore be
regenerated on its own.

Init stream, drawn in this order:
  1. V0 = Q factor (positive diagonal) of an n x r standard normal draw,
     formed in float64 and rounded to float32;
  2. X0 = x0_std * N(0,1) (m x n), rounded to float32;
  3. planted workloads only: A (m x K) and B (n x K), orthonormal the same way.
R0 is all zeros.

Step t draws Z_t (m x n standard normal) and forms G_t in float64:
  "normal":  G_t = noise * Z_t
  "planted": G_t = A diag(1/k) B^T + noise * Z_t,  k = 1..K
then rounds to float32 (round to nearest even).  bf16 workloads round that
float32 value once more to bfloat16 (round to nearest even) and hand out the
raw 16-bit patterns.

Random orthonormal factors use LAPACK's QR through numpy; that is input
preparation only.  Nothing here computes any part of the optimizer step.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .configs import MatrixSpec, Workload


def rng(seed: int, i: int, s: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(i), int(s)])


def random_orthonormal(g: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """rows x cols float64 matrix with orthonormal columns (Haar-distributed)."""
    z = g.standard_normal((rows, cols))
    q, rf = np.linalg.qr(z, mode="reduced")
    d = np.sign(np.diag(rf))
    d[d == 0] = 1.0
    return q * d


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    NaN stays NaN (quiet bit forced); infinities and overflow behave as IEEE
    rounding does.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


class MatrixStream:
    """Inputs of one matrix of a workload, addressable by step."""

    _CACHE_BYTES = 256 << 20

    def __init__(self, wl: Workload, spec: MatrixSpec):
        self.wl = wl
        self.spec = spec
        self._A: Optional[np.ndarray] = None
        self._B: Optional[np.ndarray] = None
        self._L: Optional[np.ndarray] = None
        self._init = None

    @property
    def noise(self) -> float:
        return float(self.wl.noise[self.spec.index])

    @property
    def planted_rank(self) -> int:
        k = self.wl.planted_rank
        return min(self.spec.m, self.spec.n) if k == 0 else k

    def init(self):
        """(X0 f32, R0 f32 zeros, V0 f32)."""
        if self._init is None:
            s = self.spec
            g = rng(self.wl.seed, s.index, 0)
            v0 = random_orthonormal(g, s.n, s.r).astype(np.float32)
            x0 = (self.wl.x0_std * g.standard_normal((s.m, s.n))).astype(np.float32)
            if self.wl.g_kind == "planted":
                k = self.planted_rank
                self._A = random_orthonormal(g, s.m, k)
                self._B = random_orthonormal(g, s.n, k)
            r0 = np.zeros((s.m, s.n), dtype=np.float32)
            self._init = (x0, r0, v0)
        x0, r0, v0 = self._init
        return x0.copy(), r0.copy(), v0.copy()

    def _low_rank(self) -> np.ndarray:
        if self._L is not None:
            return self._L
        if self._A is None:
            self.init()
        k = self.planted_rank
        scale = 1.0 / np.arange(1, k + 1, dtype=np.float64)
        low = (self._A * scale) @ self._B.T
        if low.nbytes <= self._CACHE_BYTES:
            self._L = low
        return low

    def grad_f32(self, t: int) -> np.ndarray:
        """G_t rounded to float32 (before any bf16 rounding)."""
        s = self.spec
        g = rng(self.wl.seed, s.index, t + 1)
        z = g.standard_normal((s.m, s.n))
        if self.wl.g_kind == "planted":
            out = self._low_rank() + self.noise * z
        else:
            out = self.noise * z
        return out.astype(np.float32)

    def grad(self, t: int) -> np.ndarray:
        """G_t as the library receives it: float32 array or uint16 bf16 bits."""
        g32 = self.grad_f32(t)
        if self.wl.g_dtype == "bf16":
            return f32_to_bf16_bits(g32)
        return g32

    def grad_f64(self, t: int) -> np.ndarray:
        """The exact value of what ``grad`` hands out, widened to float64."""
        g = self.grad(t)
        if self.wl.g_dtype == "bf16":
            return bf16_bits_to_f32(g).astype(np.float64)
        return g.astype(np.float64)


def conditioned_inputs(m: int, n: int, r: int, kappa: float, seed: int,
                       g_dtype: str = "f32", side: str = "P",
                       duplicate: Optional[int] = None):
    """One matrix whose factor P = M V (side "P") or W = M^T U (side "W")
    has nearly collinear columns and a condition number of about kappa:
    M = A diag(s) B^T with A (m x k), B (n x k) random orthonormal,
    k = min(r + 8, m, n), s log-spaced from 1 down to 1/kappa over the first
    r directions and 1/(10 kappa) on the rest; R0 = 0, X0 = 0.02 N(0,1).
    Side "P": V0 random orthonormal, so every column of P mixes all the
    directions.  Side "W": V0 = B_r diag(1/s) Z (Z random orthonormal r x r)
    with each column scaled to unit length, so P = A_r Z D is well-
    conditioned and U = orth(P) mixes the directions evenly, and W = B_r
    diag(s) Z' is the ill-conditioned factor.  duplicate = j makes column
    j + 1 of V0 a copy of column j (P then has two equal columns).  Returns
    (X0, G, R0, V0) as the library receives them (G float32 or bfloat16
    bits)."""
    g = rng(seed, 0, 0)
    k = min(r + 8, m, n)
    A = random_orthonormal(g, m, k)
    B = random_orthonormal(g, n, k)
    s = np.full(k, 0.1 / kappa)
    s[:min(r, k)] = np.logspace(0.0, -np.log10(kappa), min(r, k))
    G = ((A * s) @ B.T).astype(np.float32)
    if side == "W":
        Z = random_orthonormal(g, r, r)
        V = (B[:, :r] / s[:r]) @ Z
        V /= np.linalg.norm(V, axis=0)
    else:
        V = random_orthonormal(g, n, r)
    if duplicate is not None:
        V[:, duplicate + 1] = V[:, duplicate]
    X = (0.02 * g.standard_normal((m, n))).astype(np.float32)
    if g_dtype == "bf16":
        G = f32_to_bf16_bits(G)
    return X, G, np.zeros((m, n), dtype=np.float32), V.astype(np.float32)
