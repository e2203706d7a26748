"""Seeded inputs drawn directly on the GPU, for timing runs.

Same shapes and dtypes as the numpy recipe in generators.py, and the same
distributions for X0 = 0.02 N(0,1) and G = A diag(1/k) B^T + noise Z (or
noise Z), bf16-rounded for bf16 workloads; V0, A and B are orthonormal (see
below).  Drawn with torch's seeded device generator so that a
2.8-billion-element stack is ready in seconds.  The values differ from the
numpy streams; parity tests use the numpy streams, the benchmark uses these.

Orthonormal factors here are built without a factorization (so that the
inputs need no solver library): a random signed selection of `cols` of the
`rows` unit vectors, mixed by three random Householder reflections.  The
columns are exactly orthonormal up to float32 rounding and dense, though not
Haar-distributed; the step's cost does not depend on their values.
"""
from __future__ import annotations

import torch

from .configs import MatrixSpec, Workload


def _gen(seed: int, i: int, s: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1_000_003 + i) * 1_000_003 + s) % (2 ** 63))
    return g


def orthonormal(rows: int, cols: int, gen: torch.Generator, device) -> torch.Tensor:
    pick = torch.randperm(rows, generator=gen, device=device)[:cols]
    sign = torch.randint(0, 2, (cols,), generator=gen, device=device).float() * 2.0 - 1.0
    q = torch.zeros(rows, cols, device=device, dtype=torch.float32)
    q[pick, torch.arange(cols, device=device)] = sign
    for _ in range(3):
        u = torch.randn(rows, 1, generator=gen, device=device, dtype=torch.float32)
        u /= torch.linalg.vector_norm(u)
        q -= 2.0 * u @ (u.t() @ q)
    return q.contiguous()


class DeviceMatrix:
    """State and gradient of one matrix on the device."""

    def __init__(self, wl: Workload, spec: MatrixSpec, device, with_planted: bool = True):
        self.wl, self.spec, self.device = wl, spec, device
        g0 = _gen(wl.seed, spec.index, 0, device)
        self.V = orthonormal(spec.n, spec.r, g0, device)
        self.X = (wl.x0_std * torch.randn(spec.m, spec.n, generator=g0, device=device))
        self.R = torch.zeros(spec.m, spec.n, device=device)
        self._A = self._B = None
        if wl.g_kind == "planted" and with_planted:
            k = wl.planted_rank or min(spec.m, spec.n)
            self._A = orthonormal(spec.m, k, g0, device)
            scale = 1.0 / torch.arange(1, k + 1, device=device, dtype=torch.float32)
            self._A = self._A * scale
            self._B = orthonormal(spec.n, k, g0, device)
        self.G = self.grad(0)

    def grad(self, t: int) -> torch.Tensor:
        wl, s = self.wl, self.spec
        gen = _gen(wl.seed, s.index, t + 1, self.device)
        g = float(wl.noise[s.index]) * torch.randn(s.m, s.n, generator=gen, device=self.device)
        if self._A is not None:
            g.addmm_(self._A, self._B.t())
        if wl.g_dtype == "bf16":
            return g.to(torch.bfloat16)
        return g

    def reset_rank(self, r: int) -> None:
        """New warm start for a different rank (same matrix)."""
        g0 = _gen(self.wl.seed, self.spec.index, 10_000 + r, self.device)
        self.V = orthonormal(self.spec.n, r, g0, self.device)
