"""Shared helpers of the GPU tests: move seeded inputs to the device, run
libdion, run the oracle on the same bytes, compare."""
from __future__ import annotations

import sys

import numpy as np

from oracle import dion_step as oracle_step
from oracle.checks import rel_fro
from workloads import MatrixStream

TOL_1 = 1e-4      # relative Frobenius error after one step
TOL_LONG = 1e-3   # after the workload's full step count


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, bf16: bool = False):
    import torch
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def g_f64(g: np.ndarray, bf16: bool) -> np.ndarray:
    if bf16:
        from workloads import bf16_bits_to_f32
        return bf16_bits_to_f32(g).astype(np.float64)
    return g.astype(np.float64)


def f32(x: float) -> float:
    return float(np.float32(x))


class Case:
    """Device state of one matrix plus the float64 state the oracle tracks."""

    def __init__(self, wl, spec):
        self.wl, self.spec = wl, spec
        self.bf16 = wl.g_dtype == "bf16"
        self.stream = MatrixStream(wl, spec)
        x0, r0, v0 = self.stream.init()
        self.X, self.R, self.V = to_dev(x0), to_dev(r0), to_dev(v0)
        self.x, self.r, self.v = (a.astype(np.float64) for a in (x0, r0, v0))
        self.G = None
        self.g = None

    def load_grad(self, t: int):
        g = self.stream.grad(t)
        self.G = to_dev(g, self.bf16)
        self.g = g_f64(g, self.bf16)

    def oracle(self, variant: str, eta=None, beta=None):
        eta = f32(self.wl.eta if eta is None else eta)
        beta = f32(self.wl.beta if beta is None else beta)
        res = oracle_step(self.x, self.g, self.r, self.v, eta, beta, variant)
        x_prev = self.x
        self.x, self.r, self.v = res.X, res.R, res.V
        self.last_M = res.M
        return res, x_prev

    def errors(self, x_prev=None, M=None) -> dict:
        """Relative Frobenius errors against the oracle's state.

        When r = min(m, n), span(U) holds the whole column space of M and the
        exact residual is zero; its relative error is then undefined, so R is
        measured against ||beta M||_F instead (M: the step's buffer)."""
        X = self.X.double().cpu().numpy()
        Rg = self.R.double().cpu().numpy()
        full = self.spec.r == min(self.spec.m, self.spec.n)
        if full and M is not None:
            beta = f32(self.wl.beta)
            r_err = float(np.linalg.norm(Rg - self.r) / max(beta * np.linalg.norm(M), 1e-300))
        else:
            r_err = rel_fro(Rg, self.r)
        out = {"X": rel_fro(X, self.x), "R": r_err,
               "V": rel_fro(self.V.double().cpu().numpy(), self.v)}
        if x_prev is not None:
            out["dX"] = rel_fro(X - x_prev, self.x - x_prev)
        return out


def assert_close(err: dict, tol: float, what: str = ""):
    bad = {k: v for k, v in err.items() if not v <= tol}
    assert not bad, f"{what}: relative Frobenius errors above {tol}: {err}"
