"""The one-workgroup step of small matrices (k_small) against the oracle (GPU).

Matrices with r <= 16 whose factors fit the kernel's LDS and whose products
are at most 2^21 multiply-adds take the whole step in one launch
(include/dion.h, DION_SCHED_GROUPED).  These tests hold that path to the
same bar as the grouped schedule: relative Frobenius error <= 1e-4 on X, R,
V and dX after one step against the float64 oracle (Orth-Dion page,
equation block), on shapes that exercise each of its loops (several row
sets of M V, several column sets of M^T U and of the update, rows of one
to 900 columns, rank blocks 8 and 16), and the same inputs through the
grouped schedule for comparison.  Ill-conditioned factors, breakdowns and
mixed plans (small and grouped classes in one call) are covered as well."""
import numpy as np
import pytest

from oracle import DION, ORTH, Breakdown, qr_pos
from oracle.checks import rel_fro
from workloads import conditioned_inputs
from workloads.configs import MatrixSpec, Workload

from .gpuhelp import TOL_1, Case, assert_close, say

pytestmark = pytest.mark.gpu

# the library's admission rule for the one-workgroup step, and whether it
# keeps M resident in LDS
def small_path(m, n, r):
    rb = 8 if r <= 8 else 16 if r <= 16 else 0
    n32 = (n + 31) // 32 * 32
    return rb > 0 and (m + n + n32) * rb <= 16384 and m * n * r <= 1 << 21


def resident(m, n, r):
    rb = 8 if r <= 8 else 16
    n32 = (n + 31) // 32 * 32
    return small_path(m, n, r) and m * (n + 1) + (m + n32) * (rb + 1) <= 39680


SMALL = [(256, 128, 16), (131, 67, 3), (1, 7, 1), (9, 1, 1), (64, 48, 16), (200, 100, 9),
         (600, 150, 8), (100, 900, 6), (260, 300, 16), (40, 250, 13)]


def _wl(m, n, r, g_dtype="f32", seed=101):
    return Workload(name=f"s{m}x{n}r{r}", seed=seed, mats=(MatrixSpec(0, "W", 0, m, n, r),),
                    g_dtype=g_dtype, g_kind="normal", noise=(1.0,), planted_rank=0,
                    eta=0.01, beta=0.95, steps=1, variants=("orth", "dion"))


def test_shapes_take_the_small_path():
    assert all(small_path(*s) for s in SMALL)
    assert not small_path(257, 129, 17) and not small_path(1000, 37, 20)
    # both forms of the kernel are covered
    assert sum(resident(*s) for s in SMALL) >= 4 and sum(not resident(*s) for s in SMALL) >= 3


@pytest.mark.parametrize("m,n,r", SMALL)
@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("g_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("sched", ["small", "grouped"])
def test_small_shapes(gpu_lib, m, n, r, variant, g_dtype, sched):
    wl = _wl(m, n, r, g_dtype, seed=200 + m + n + r)
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    say(f"small {m}x{n} r={r} {variant} {g_dtype} {sched}")
    math = gpu_lib.MATH["f32"] | (gpu_lib.SCHED_GROUPED if sched == "grouped" else 0)
    ws = gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, variant, math=math)
    assert gpu_lib.status(ws, 1)[0] == 0
    res, x_prev = c.oracle(variant)
    assert_close(c.errors(x_prev, res.M), TOL_1, f"small {m}x{n} r={r} {variant} {g_dtype} {sched}")


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_small_is_deterministic_and_repeatable(gpu_lib, variant):
    import torch
    wl = _wl(260, 300, 16) if variant == ORTH else _wl(256, 128, 16)
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    s0 = [t.clone() for t in (c.X, c.R, c.V)]
    outs = []
    for _ in range(2):
        for dst, src in zip((c.X, c.R, c.V), s0):
            dst.copy_(src)
        gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, variant)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (c.X, c.R, c.V)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("kappa", [1e4, 1e6])
@pytest.mark.parametrize("side", ["P", "W"])
@pytest.mark.parametrize("variant", ["orth", "dion"])
@pytest.mark.parametrize("m,n,r", [(200, 120, 12), (600, 150, 12)])
def test_small_ill_conditioned(gpu_lib, kappa, side, variant, m, n, r):
    # the second pass and the shifted retry inside the one-workgroup step
    # (resident and streaming forms): every stage against its definition on
    # the kernel's own float32 inputs
    from .test_gpu_orth_range import CTL_RETRY, CTL_TWO, _check_stages, _run
    assert small_path(m, n, r)
    case = conditioned_inputs(m, n, r, kappa, seed=int(7 * r + np.log10(kappa)), side=side)
    what = f"small {m}x{n} r={r} kappa={kappa:.0e} ({side}) {variant}"
    say(what)
    rc, per, raw, out = _run(gpu_lib, [case], variant, "f32")
    assert rc == 0, (what, per)
    if (side == "W") == (variant == "orth"):
        assert raw[0] & CTL_TWO, (what, hex(raw[0]))
        if kappa >= 1e6:
            assert raw[0] & CTL_RETRY, (what, hex(raw[0]))
    _check_stages(case, out[0], variant, "f32", what)


@pytest.mark.parametrize("variant", ["orth", "dion"])
@pytest.mark.parametrize("m,n,r", [(200, 120, 12), (600, 150, 12)])
def test_small_dependent_columns_break_down(gpu_lib, variant, m, n, r):
    import torch
    X, G, R, V = conditioned_inputs(m, n, r, 10.0, seed=23, duplicate=4)
    with pytest.raises(Breakdown):
        qr_pos(G.astype(np.float64) @ V.astype(np.float64))
    Xd, Gd, Rd, Vd = (torch.from_numpy(a.copy()).cuda() for a in (X, G, R, V))
    ws = gpu_lib.step(Xd, Gd, Rd, Vd, 0.01, 0.95, variant)
    rc, per = gpu_lib.status(ws, 1)
    assert rc == gpu_lib.ERR_BREAKDOWN and per[0] & gpu_lib.STATUS_ORTH_P, per
    for dev, host in ((Xd, X), (Rd, R), (Vd, V)):
        assert np.array_equal(dev.cpu().numpy(), host)


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_plan_mixing_small_and_grouped_classes(gpu_lib, variant):
    # one call whose small classes take k_small and whose others take the
    # grouped launches; the intermediate factors of both are readable
    shapes = [(256, 128, 16), (256, 192, 48), (100, 900, 6), (300, 200, 40), (256, 128, 16)]
    cases = [Case(_wl(m, n, r, seed=300 + i), MatrixSpec(0, "W", 0, m, n, r))
             for i, (m, n, r) in enumerate(shapes)]
    for c in cases:
        c.load_grad(0)
    say(f"mixed small and grouped {variant}")
    plan = gpu_lib.Plan([(c.X, c.G, c.R, c.V) for c in cases], variant)
    ws = plan.new_workspace()
    plan.step(0.01, 0.95, ws)
    assert gpu_lib.status(ws, plan.count)[0] == 0
    for i, (c, (m, n, r)) in enumerate(zip(cases, shapes)):
        U = plan.buffer(ws, gpu_lib.BUF_U, i).double().cpu().numpy()
        P = plan.buffer(ws, gpu_lib.BUF_P, i).double().cpu().numpy()
        assert rel_fro(U, qr_pos(P)[0]) < 1e-5, (m, n, r)
        res, xp = c.oracle(variant)
        assert_close(c.errors(xp, res.M), TOL_1, f"mixed {m}x{n} r={r} {variant}")
    plan.close()
