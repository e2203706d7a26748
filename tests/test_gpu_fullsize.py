"""libdion at the workloads' full sizes (GPU).

* The 3B Llama-shaped stack, all 196 matrices in one grouped step through a
  plan (the launch configuration the benchmark times), in both arithmetics:
  one matrix of each of the four shapes in the first and in the last layer
  is fed the seeded numpy streams and checked against the float64 oracle;
  every matrix is checked for the step's invariants and for its residual
  R' = beta (M - U W^T) on a sample of rows and columns, formed from its own
  U (read back from the workspace) and full rows and columns of M.
* A stack of 128 ragged 2100 x 2060 matrices at r = 150, large enough for
  the 256 x 192 split-bfloat16 product tiles, sampled against the oracle.
* The 8192 x 28672 matrix at rank 2048 (Orth-Dion), one step against the
  full float64 oracle.
The long horizons are in test_gpu_horizon.py.
"""
import math

import numpy as np
import pytest

from oracle import ORTH, DION
from oracle.checks import rel_fro, sampled_residual
from workloads import config

from .gpuhelp import TOL_1, Case, assert_close, f32, say

pytestmark = pytest.mark.gpu

# one matrix of each shape class (Q 3072x3072, K 3072x1024, gate 3072x8192,
# down 8192x3072) in layer 0 and in layer 27
SAMPLED = (0, 1, 4, 6, 189, 190, 193, 195)


def _stack(wl, sampled):
    import torch
    from workloads.device import DeviceMatrix
    dev = torch.device("cuda", 0)
    mats, cases = [], {}
    for s in wl.mats:
        if s.index in sampled:
            c = Case(wl, s)
            c.load_grad(0)
            cases[s.index] = c
            mats.append((c.X, c.G, c.R, c.V))
        else:
            d = DeviceMatrix(wl, s, dev)
            mats.append((d.X, d.G, d.R, d.V))
    return mats, cases


def _residual_sample(spec, G, R_new, U, beta, seed):
    """Relative error of R' on 16 rows x 16 columns of one matrix: the
    oracle's sampled_residual from full rows and columns of M = G (R0 = 0)
    and the library's own U."""
    g = np.random.default_rng(seed)
    rows = np.sort(g.choice(spec.m, size=16, replace=False))
    cols = np.sort(g.choice(spec.n, size=16, replace=False))
    Gd = G.double()
    m_rows = Gd[rows].cpu().numpy()
    m_cols = Gd[:, cols].cpu().numpy()
    ref = sampled_residual(m_rows, m_cols, U, rows, cols, beta)
    got = R_new.double()[rows][:, cols].cpu().numpy()
    return rel_fro(got, ref)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("rank_div", [4, 16])
def test_config4_full_stack(gpu_lib, variant, rank_div):
    import torch
    wl = config(4, rank_div)
    say(f"config4 r=1/{rank_div} {variant}: building 196 matrices")
    mats, cases = _stack(wl, SAMPLED)
    x0 = [m[0].clone() for m in mats]
    v0 = [m[3].clone() for m in mats]
    refs = {}
    for idx, c in cases.items():
        say(f"config4: oracle on matrix {idx} ({c.spec.m}x{c.spec.n} r={c.spec.r})")
        refs[idx] = c.oracle(variant)
    eta, beta = f32(wl.eta), f32(wl.beta)
    for arith in ("f32", "bf16x3"):
        for (X, G, R, V), xs, vs in zip(mats, x0, v0):
            X.copy_(xs)
            R.zero_()
            V.copy_(vs)
        plan = gpu_lib.Plan(mats, variant, math=arith)
        ws = plan.new_workspace()
        plan.step(wl.eta, wl.beta, ws)
        rc, per = gpu_lib.status(ws, plan.count)
        assert rc == 0, per
        say(f"config4 r=1/{rank_div} {variant} {arith}: invariants and residual samples of all 196")
        worst_r = 0.0
        for s, (X, G, R, V), xp in zip(wl.mats, mats, x0):
            dx = (xp.double() - X.double())
            assert abs(torch.linalg.norm(dx).item() - eta * math.sqrt(s.r)) < 1e-3 * eta * math.sqrt(s.r)
            Vd = V.double()
            if variant == ORTH:
                err = (Vd.T @ Vd - torch.eye(s.r, device=Vd.device, dtype=Vd.dtype)).abs().max().item()
                assert err < 1e-4, (s.index, err)
            else:
                err = (torch.linalg.norm(Vd, dim=0) - 1.0).abs().max().item()
                assert err < 1e-5, (s.index, err)
            U = plan.buffer(ws, gpu_lib.BUF_U, s.index).double().cpu().numpy()
            e = _residual_sample(s, G, R, U, beta, seed=s.index)
            worst_r = max(worst_r, e)
            assert e <= 1e-4, (s.index, arith, e)
        say(f"  worst sampled residual error {worst_r:.2e}")
        for idx, c in cases.items():
            res, x_prev = refs[idx]
            X = c.X.double().cpu().numpy()
            err = {"X": rel_fro(X, res.X), "R": rel_fro(c.R.double().cpu().numpy(), res.R),
                   "V": rel_fro(c.V.double().cpu().numpy(), res.V),
                   "dX": rel_fro(X - x_prev, res.X - x_prev)}
            say(f"  matrix {idx} {arith}: {err}")
            assert_close(err, TOL_1, f"config4 matrix {idx} {variant} {arith}")
        plan.close()
        del ws


@pytest.mark.timeout(400)
@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("r", [150, 152])
def test_wide_tiles_ragged_stack(gpu_lib, variant, r):
    """128 matrices of 2100 x 2060 at r = 150 or 152 in one split-bfloat16
    grouped step: 1,152 tiles per product launch, so M V and M^T U take the
    256 x 192 tiles, with every edge ragged (rows past 2100 and 2060,
    reduction lengths that are not multiples of 32, idle columns past r);
    r = 152 keeps 16-byte rows (the vector loads), r = 150 does not.
    Matrices 0, 63 and 127 take the seeded numpy streams and are checked
    against the float64 oracle; every matrix is checked for the step's
    invariants."""
    import torch
    from workloads import MatrixSpec, Workload
    from workloads.device import DeviceMatrix
    m, n, count = 2100, 2060, 128
    wl = Workload(name="wide-tiles-ragged", seed=77,
                  mats=tuple(MatrixSpec(i, "W", i, m, n, r) for i in range(count)),
                  g_dtype="f32", g_kind="normal", noise=(1.0,) * count, planted_rank=0,
                  eta=0.01, beta=0.95, steps=1, variants=("orth", "dion"))
    sampled = (0, 63, 127)
    dev = torch.device("cuda", 0)
    mats, cases = [], {}
    for s in wl.mats:
        if s.index in sampled:
            c = Case(wl, s)
            c.load_grad(0)
            cases[s.index] = c
            mats.append((c.X, c.G, c.R, c.V))
        else:
            d = DeviceMatrix(wl, s, dev)
            mats.append((d.X, d.G, d.R, d.V))
    x0 = [t[0].clone() for t in mats]
    say(f"wide tiles {variant}: one grouped split-bfloat16 step over {count} matrices")
    plan = gpu_lib.Plan(mats, variant, math="bf16x3")
    ws = plan.new_workspace()
    plan.step(wl.eta, wl.beta, ws)
    rc, per = gpu_lib.status(ws, plan.count)
    assert rc == 0, per
    eta = f32(wl.eta)
    for s, (X, G, R, V), xp in zip(wl.mats, mats, x0):
        dx = torch.linalg.norm(xp.double() - X.double()).item()
        assert abs(dx - eta * math.sqrt(r)) < 1e-3 * eta * math.sqrt(r), (s.index, dx)
        Vd = V.double()
        if variant == ORTH:
            err = (Vd.T @ Vd - torch.eye(r, device=Vd.device, dtype=Vd.dtype)).abs().max().item()
            assert err < 1e-4, (s.index, err)
        else:
            err = (torch.linalg.norm(Vd, dim=0) - 1.0).abs().max().item()
            assert err < 1e-5, (s.index, err)
    for idx, c in cases.items():
        say(f"wide tiles {variant}: oracle on matrix {idx}")
        res, x_prev = c.oracle(variant)
        X = c.X.double().cpu().numpy()
        err = {"X": rel_fro(X, res.X), "R": rel_fro(c.R.double().cpu().numpy(), res.R),
               "V": rel_fro(c.V.double().cpu().numpy(), res.V),
               "dX": rel_fro(X - x_prev, res.X - x_prev)}
        say(f"  matrix {idx}: {err}")
        assert_close(err, TOL_1, f"wide tiles matrix {idx} {variant}")
    plan.close()
    del ws


@pytest.mark.timeout(400)
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_config5_rank2048_one_step(gpu_lib, arith):
    wl = config(5, r=2048)
    say(f"config5 r=2048 {arith}: inputs")
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, ORTH, math=arith)
    say("config5 r=2048: float64 oracle")
    _, x_prev = c.oracle(ORTH)
    assert_close(c.errors(x_prev), TOL_1, "config5 r=2048")
