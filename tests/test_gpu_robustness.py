"""Breakdown handling, determinism and resume of libdion (GPU)."""
import numpy as np
import pytest

from oracle import ORTH
from workloads import config
from workloads.configs import MatrixSpec, Workload

from .gpuhelp import Case, say

pytestmark = pytest.mark.gpu
ARITH = pytest.mark.parametrize("arith", ["f32", "bf16x3"])


def _case(m=300, n=200, r=40, g_dtype="f32", seed=5):
    wl = Workload(name="rb", seed=seed, mats=(MatrixSpec(0, "W", 0, m, n, r),), g_dtype=g_dtype,
                  g_kind="normal", noise=(1.0,), planted_rank=0, eta=0.01, beta=0.95, steps=1,
                  variants=("orth", "dion"))
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    return c


def _snap(c):
    return c.X.clone(), c.R.clone(), c.V.clone()


def _same(a, b):
    import torch
    return all(torch.equal(u, w) for u, w in zip(a, b))


@ARITH
@pytest.mark.parametrize("variant", ["orth", "dion"])
def test_zero_buffer_breaks_down_and_leaves_state(gpu_lib, variant, arith):
    c = _case()
    c.G.zero_()
    c.R.zero_()
    before = _snap(c)
    say(f"breakdown zero buffer {variant} {arith}")
    ws = gpu_lib.step(c.X, c.G, c.R, c.V, 0.01, 0.95, variant, math=arith)
    rc, per = gpu_lib.status(ws, 1)
    assert rc == gpu_lib.ERR_BREAKDOWN and per[0] & gpu_lib.STATUS_ORTH_P
    assert _same(before, _snap(c))
    with pytest.raises(gpu_lib.Breakdown):
        gpu_lib.check_status(ws, 1)


@ARITH
@pytest.mark.parametrize("variant", ["orth", "dion"])
def test_nan_gradient_breaks_down(gpu_lib, variant, arith):
    c = _case(g_dtype="bf16")
    import torch
    c.G[3, 7] = torch.nan
    before = _snap(c)
    ws = gpu_lib.step(c.X, c.G, c.R, c.V, 0.01, 0.95, variant, math=arith)
    rc, per = gpu_lib.status(ws, 1)
    assert rc == gpu_lib.ERR_BREAKDOWN and per[0] != 0
    assert _same(before, _snap(c))


@ARITH
def test_status_resets_after_breakdown(gpu_lib, arith):
    """A step after a breakdown, on the same workspace, runs every phase
    again and matches a step on a fresh workspace bit for bit."""
    c = _case()
    g = c.G.clone()
    c.G.zero_()
    r = c.R.clone()
    c.R.zero_()
    ws = gpu_lib.step(c.X, c.G, c.R, c.V, 0.01, 0.95, "orth", math=arith)
    assert gpu_lib.status(ws, 1)[0] == gpu_lib.ERR_BREAKDOWN
    c.G.copy_(g)
    c.R.copy_(r)
    s0 = _snap(c)
    gpu_lib.step(c.X, c.G, c.R, c.V, 0.01, 0.95, "orth", workspace=ws, math=arith)
    assert gpu_lib.status(ws, 1) == (0, [0])
    s1 = _snap(c)
    c.X.copy_(s0[0])
    c.R.copy_(s0[1])
    c.V.copy_(s0[2])
    gpu_lib.step(c.X, c.G, c.R, c.V, 0.01, 0.95, "orth", math=arith)
    assert _same(s1, _snap(c))


@ARITH
def test_batched_breakdown_is_per_matrix(gpu_lib, arith):
    a, b = _case(seed=1), _case(seed=2)
    b.G.zero_()
    b.R.zero_()
    sa, sb = _snap(a), _snap(b)
    ws = gpu_lib.step_batched([(a.X, a.G, a.R, a.V), (b.X, b.G, b.R, b.V)], 0.01, 0.95, "orth",
                              math=arith)
    rc, per = gpu_lib.status(ws, 2)
    assert rc == gpu_lib.ERR_BREAKDOWN and per[0] == 0 and per[1] != 0
    assert _same(sb, _snap(b))
    assert not _same(sa, _snap(a))


@ARITH
@pytest.mark.parametrize("variant", ["orth", "dion"])
def test_bitwise_deterministic(gpu_lib, variant, arith):
    c = _case(700, 900, 130)
    s0 = _snap(c)
    gpu_lib.step(c.X, c.G, c.R, c.V, 0.01, 0.95, variant, math=arith)
    s1 = _snap(c)
    c.X.copy_(s0[0])
    c.R.copy_(s0[1])
    c.V.copy_(s0[2])
    gpu_lib.step(c.X, c.G, c.R, c.V, 0.01, 0.95, variant, math=arith)
    assert _same(s1, _snap(c))


@ARITH
def test_resume_from_saved_state_is_bitwise(gpu_lib, arith):
    wl = config(1)
    c = Case(wl, wl.mats[0])
    grads = []
    for t in range(6):
        c.load_grad(t)
        grads.append(c.G)
    init = _snap(c)
    for g in grads:
        gpu_lib.step(c.X, g, c.R, c.V, wl.eta, wl.beta, ORTH, math=arith)
    straight = _snap(c)
    c.X.copy_(init[0])
    c.R.copy_(init[1])
    c.V.copy_(init[2])
    for g in grads[:3]:
        gpu_lib.step(c.X, g, c.R, c.V, wl.eta, wl.beta, ORTH, math=arith)
    saved = [t.cpu().numpy().copy() for t in _snap(c)]
    c.X.fill_(np.nan)
    c.R.fill_(np.nan)
    c.V.fill_(np.nan)
    import torch
    for dst, src in zip((c.X, c.R, c.V), saved):
        dst.copy_(torch.from_numpy(src).cuda())
    for g in grads[3:]:
        gpu_lib.step(c.X, g, c.R, c.V, wl.eta, wl.beta, ORTH, math=arith)
    assert _same(straight, _snap(c))
