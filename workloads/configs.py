"""The five synthetic workloads the step is tested and measured on.

Shapes follow the model sizes the Dion abstract evaluates on (language models
from 160M to 3B parameters, "Dion: Distributed Orthonormalized Updates",
Abstract) plus a single small matrix, a single planted-spectrum matrix and one
70B-style MLP projection.  Every matrix is m x n with m rows and n columns,
taken literally (no automatic transpose).

Matrix order inside a stack is layer-major; inside a layer the roles come in
the order listed in ``roles``.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple


@dataclasses.dataclass(frozen=True)
class MatrixSpec:
    """One weight matrix of a workload."""
    index: int          # position in the stack; also the random-stream index
    role: str           # "Q", "K", ..., or "W" for single-matrix workloads
    layer: int
    m: int
    n: int
    r: int


@dataclasses.dataclass(frozen=True)
class Workload:
    """A workload: a list of matrices plus the recipe for G, X0 and V0.

    g_kind:
      "normal"  G = noise * Z
      "planted" G = A diag(1/k) B^T + noise * Z, A (m x K), B (n x K) random
                orthonormal, k = 1..K
    Z is a fresh standard normal draw at every step.
    """
    name: str
    seed: int
    mats: Tuple[MatrixSpec, ...]
    g_dtype: str            # "f32" or "bf16"
    g_kind: str             # "normal" or "planted"
    noise: Tuple[float, ...]  # per-matrix noise scale on Z
    planted_rank: int       # K for "planted" (0 = min(m, n))
    eta: float
    beta: float
    steps: int
    variants: Tuple[str, ...]
    x0_std: float = 0.02

    @property
    def count(self) -> int:
        return len(self.mats)

    @property
    def elements(self) -> int:
        return sum(s.m * s.n for s in self.mats)


def _single(name, seed, m, n, r, g_dtype, g_kind, noise, planted_rank, eta,
            beta, steps, variants) -> Workload:
    return Workload(name=name, seed=seed,
                    mats=(MatrixSpec(0, "W", 0, m, n, r),),
                    g_dtype=g_dtype, g_kind=g_kind, noise=(noise,),
                    planted_rank=planted_rank, eta=eta, beta=beta, steps=steps,
                    variants=variants)


def stack_160m(layers: int = 12) -> List[Tuple[str, int, int]]:
    """GPT-shaped 160M stack: d = 768, MLP width 3072."""
    d, f = 768, 3072
    roles = [("Q", d, d), ("K", d, d), ("V", d, d), ("O", d, d),
             ("up", d, f), ("down", f, d)]
    return [(name, m, n) for _ in range(layers) for (name, m, n) in roles]


def stack_3b(layers: int = 28) -> List[Tuple[str, int, int]]:
    """Llama-shaped 3B stack: hidden 3072, GQA K/V 3072 x 1024, MLP 8192."""
    h, kv, f = 3072, 1024, 8192
    roles = [("Q", h, h), ("K", h, kv), ("V", h, kv), ("O", h, h),
             ("gate", h, f), ("up", h, f), ("down", f, h)]
    return [(name, m, n) for _ in range(layers) for (name, m, n) in roles]


def _stack(shapes, per_layer, frac) -> Tuple[MatrixSpec, ...]:
    out = []
    for i, (role, m, n) in enumerate(shapes):
        r = min(m, n) // frac
        out.append(MatrixSpec(i, role, i // per_layer, m, n, r))
    return tuple(out)


def config(num: int, rank_div: int = 4, r: Optional[int] = None,
           layers: Optional[int] = None) -> Workload:
    """Return workload ``num`` (1..5).

    rank_div: rank fraction denominator for the stacks (4 or 16).
    r:        rank for config 5 (512 or 2048).
    layers:   optional layer count override for the stacks (sampling only).
    """
    both = ("dion", "orth")
    if num == 1:
        return _single("single-256x128-r16", 1, 256, 128, 16, "f32", "normal",
                       1.0, 0, 0.01, 0.95, 10, both)
    if num == 2:
        return _single("planted-2048x2048-r512", 2, 2048, 2048, 512, "f32",
                       "planted", 0.01, 0, 0.02, 0.95, 100, both)
    if num == 3:
        shapes = stack_160m(layers or 12)
        mats = _stack(shapes, 6, 4)
        return Workload(name="gpt160m-stack-r1/4", seed=3, mats=mats,
                        g_dtype="f32", g_kind="normal",
                        noise=tuple(1.0 / (s.n ** 0.5) for s in mats),
                        planted_rank=0, eta=0.01, beta=0.95, steps=100,
                        variants=both)
    if num == 4:
        shapes = stack_3b(layers or 28)
        mats = _stack(shapes, 7, rank_div)
        return Workload(name=f"llama3b-stack-r1/{rank_div}", seed=4, mats=mats,
                        g_dtype="bf16", g_kind="planted",
                        noise=tuple(1e-3 for _ in mats), planted_rank=64,
                        eta=0.01, beta=0.95, steps=100, variants=both)
    if num == 5:
        rr = 512 if r is None else r
        return _single(f"mlp70b-8192x28672-r{rr}", 5, 8192, 28672, rr, "bf16",
                       "normal", 1.0 / (28672 ** 0.5), 0, 0.01, 0.95, 20,
                       ("orth", "dion"))
    raise ValueError(f"unknown config {num}")


CONFIGS = {
    1: lambda: config(1),
    2: lambda: config(2),
    3: lambda: config(3),
    4: lambda: config(4, 4),
    "4/16": lambda: config(4, 16),
    5: lambda: config(5, r=512),
    "5/2048": lambda: config(5, r=2048),
}
