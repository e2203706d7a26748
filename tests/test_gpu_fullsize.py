"""libdion at the workloads' full sizes (GPU).

* The 3B Llama-shaped stack, all 196 matrices in one grouped step through a
  plan (the launch configuration the benchmark times): one matrix of each
  of the four shapes is fed the seeded numpy streams and checked against
  the float64 oracle; every matrix is checked for the step's invariants.
* The 8192 x 28672 matrix at rank 2048 (Orth-Dion), one step against the
  full float64 oracle.
* The planted 2048 x 2048 matrix over 100 steps: the trajectory is compared
  with the oracle at every horizon, against the divergence that rounding
  the state to float32 alone produces in the oracle (the float32-state
  floor), and the invariants are checked at the last step.
"""
import math

import numpy as np
import pytest

from oracle import ORTH, DION, dion_step as oracle_step
from oracle.checks import rel_fro
from workloads import MatrixStream, config

from .gpuhelp import TOL_1, Case, assert_close, f32, say, to_dev

pytestmark = pytest.mark.gpu


def _stack_case(wl, sampled):
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


@pytest.mark.timeout(300)
@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("rank_div", [4, 16])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_config4_full_stack(gpu_lib, variant, rank_div, arith):
    import torch
    wl = config(4, rank_div)
    sampled = (0, 1, 4, 6)      # layer 0: Q, K, gate, down (the four shapes)
    say(f"config4 r=1/{rank_div} {variant} {arith}: building 196 matrices")
    mats, cases = _stack_case(wl, sampled)
    x0 = [m[0].clone() for m in mats]
    plan = gpu_lib.Plan(mats, variant, math=arith)
    ws = plan.new_workspace()
    plan.step(wl.eta, wl.beta, ws)
    rc, per = gpu_lib.status(ws, plan.count)
    plan.close()
    assert rc == 0, per
    say("config4: invariants of all 196 matrices")
    eta = f32(wl.eta)
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
    for idx, c in cases.items():
        say(f"config4: oracle on matrix {idx} ({c.spec.m}x{c.spec.n} r={c.spec.r})")
        _, x_prev = c.oracle(variant)
        assert_close(c.errors(x_prev), TOL_1, f"config4 matrix {idx} {variant}")


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


# How far one step's arithmetic may exceed the error of rounding the state
# to float32 alone, on this chaotic trajectory (measured: about 17x for
# float32 products, a few hundred x for split-bfloat16's 2^-16 products).
FLOOR_FACTOR = {"f32": 100.0, "bf16x3": 1000.0}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_config2_trajectory_100_steps(gpu_lib, arith):
    wl = config(2)
    c = Case(wl, wl.mats[0])
    x_init = c.x.copy()
    eta, beta = f32(wl.eta), f32(wl.beta)
    floor_state = [c.x.copy(), c.r.copy(), c.v.copy()]
    r32 = lambda a: a.astype(np.float32).astype(np.float64)
    log = []
    for t in range(wl.steps):
        c.load_grad(t)
        gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, ORTH, math=arith)
        res, _ = c.oracle(ORTH)
        fr = oracle_step(floor_state[0], c.g, floor_state[1], floor_state[2], eta, beta, ORTH)
        floor_state = [r32(fr.X), r32(fr.R), r32(fr.V)]
        if t in (0, 4, 9, 19, 29, 39, 49, 99):
            e = c.errors(x_init)
            fl = {"X": rel_fro(floor_state[0], c.x), "R": rel_fro(floor_state[1], c.r),
                  "V": rel_fro(floor_state[2], c.v),
                  "dX": rel_fro(floor_state[0] - x_init, c.x - x_init)}
            log.append((t + 1, e, fl))
            say(f"{arith} step {t + 1}: gpu {e}  float32-state floor {fl}")
            for k in e:
                # One step's arithmetic costs a fixed multiple of the error
                # of rounding the state alone; both then grow alike.
                assert e[k] <= max(TOL_1, FLOOR_FACTOR[arith] * fl[k]), (t + 1, k, e[k], fl[k])
    # invariants still hold at the end of the trajectory
    V = c.V.double().cpu().numpy()
    assert np.max(np.abs(V.T @ V - np.eye(V.shape[1]))) < 1e-4
    assert log[0][1]["V"] <= TOL_1
