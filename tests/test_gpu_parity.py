"""libdion against the float64 oracle on the same seeded inputs (GPU).

The bar: relative Frobenius error <= 1e-4 on X, R, V and on the weight
change dX after one step, <= 1e-3 after a workload's full step count, with
float32 state.  Sizes span several 128-wide tiles and ragged tails."""
import numpy as np
import pytest

from oracle import DION, ORTH, dion_step as oracle_step
from oracle.checks import rel_fro
from workloads import config
from workloads.configs import MatrixSpec, Workload

from .gpuhelp import TOL_1, TOL_LONG, Case, assert_close, f32, g_f64, say, to_dev

pytestmark = pytest.mark.gpu


def _wl(m, n, r, g_dtype="f32", kind="normal", noise=1.0, seed=101, K=0):
    return Workload(name=f"t{m}x{n}r{r}", seed=seed, mats=(MatrixSpec(0, "W", 0, m, n, r),),
                    g_dtype=g_dtype, g_kind=kind, noise=(noise,), planted_rank=K,
                    eta=0.01, beta=0.95, steps=1, variants=("orth", "dion"))


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_config1_one_step(gpu_lib, variant):
    wl = config(1)
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    say(f"config1 {variant} one step")
    gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, variant)
    _, x_prev = c.oracle(variant)
    assert_close(c.errors(x_prev), TOL_1, f"config1 {variant}")


@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_config1_ten_steps(gpu_lib, variant, arith):
    wl = config(1)
    c = Case(wl, wl.mats[0])
    for t in range(wl.steps):
        c.load_grad(t)
        gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, variant, math=arith)
        _, x_prev = c.oracle(variant)
        assert_close(c.errors(x_prev), TOL_LONG if t else TOL_1, f"config1 {variant} step {t}")


SHAPES = [
    (257, 129, 17), (129, 257, 33), (300, 200, 100), (64, 64, 64), (200, 96, 96),
    (1, 7, 1), (9, 1, 1), (131, 67, 3), (512, 384, 128), (130, 390, 65), (1000, 37, 20),
    # ranks that take the 256 x 256 split-bfloat16 M V tiles, ragged in m, n and r
    (700, 300, 250), (520, 1000, 480),
    # odd numbers of 64-wide Cholesky blocks (3 and 5): the look-ahead pairs
    # end with an unpaired block step
    (400, 300, 150), (700, 650, 300),
]


@pytest.mark.parametrize("m,n,r", SHAPES)
@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("g_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_ragged_shapes(gpu_lib, m, n, r, variant, g_dtype, arith):
    # the grouped schedule's kernels on every shape (small ones included:
    # their own one-workgroup step is tested in test_gpu_small.py)
    wl = _wl(m, n, r, g_dtype)
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    say(f"ragged {m}x{n} r={r} {variant} {g_dtype} {arith}")
    gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, variant,
                 math=gpu_lib.MATH[arith] | gpu_lib.SCHED_GROUPED)
    res, x_prev = c.oracle(variant)
    assert_close(c.errors(x_prev, res.M), TOL_1, f"{m}x{n} r={r} {variant} {g_dtype}")


@pytest.mark.parametrize("variant", [ORTH, DION])
def test_nonzero_residual_and_second_step(gpu_lib, variant):
    # Two steps so that R != 0 and V != V0 enter the second one.
    wl = _wl(640, 520, 96, "f32", "planted", 0.05, seed=7, K=40)
    c = Case(wl, wl.mats[0])
    for t in range(2):
        c.load_grad(t)
        gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, variant)
        _, x_prev = c.oracle(variant)
        assert_close(c.errors(x_prev), TOL_1, f"planted step {t}")


@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_config2_one_step(gpu_lib, variant, arith):
    wl = config(2)
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    say(f"config2 {variant} {arith} one step")
    gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, variant, math=arith)
    _, x_prev = c.oracle(variant)
    assert_close(c.errors(x_prev), TOL_1, f"config2 {variant}")


@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
@pytest.mark.parametrize("wl_shape", ["config2", "ragged"])
def test_float64_gram_option(gpu_lib, variant, arith, wl_shape):
    # DION_GRAM_F64: the Gram matrix on the float64 matrix cores instead of
    # the sliced int8 products (the default everywhere else in this file)
    wl = config(2) if wl_shape == "config2" else _wl(400, 300, 150)
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    say(f"{wl_shape} {variant} {arith} float64 Gram one step")
    gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, variant,
                 math=gpu_lib.MATH[arith] | gpu_lib.GRAM_F64)
    _, x_prev = c.oracle(variant)
    assert_close(c.errors(x_prev), TOL_1, f"{wl_shape} {variant} float64 Gram")


@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_config5_r512_one_step(gpu_lib, arith):
    wl = config(5, r=512)
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    say(f"config5 r=512 orth {arith} one step")
    gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, ORTH, math=arith)
    _, x_prev = c.oracle(ORTH)
    assert_close(c.errors(x_prev), TOL_1, "config5 r=512")


@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_batched_config3_stack(gpu_lib, arith):
    # All 72 matrices of the 160M stack in one grouped call.
    wl = config(3)
    cases = [Case(wl, s) for s in wl.mats]
    for c in cases:
        c.load_grad(0)
    for variant in (ORTH, DION):
        say(f"config3 stack {variant} {arith}")
        state = [(c.X.clone(), c.R.clone(), c.V.clone()) for c in cases]
        gpu_lib.step_batched([(c.X, c.G, c.R, c.V) for c in cases], wl.eta, wl.beta, variant,
                             math=arith)
        worst = {}
        for c, (x0, r0, v0) in zip(cases, state):
            res = oracle_step(c.x, c.g, c.r, c.v, f32(wl.eta), f32(wl.beta), variant)
            X = c.X.double().cpu().numpy()
            err = {"X": rel_fro(X, res.X), "R": rel_fro(c.R.double().cpu().numpy(), res.R),
                   "V": rel_fro(c.V.double().cpu().numpy(), res.V),
                   "dX": rel_fro(X - c.x, res.X - c.x)}
            for k, v in err.items():
                worst[k] = max(worst.get(k, 0.0), v)
            c.X.copy_(x0)
            c.R.copy_(r0)
            c.V.copy_(v0)
        assert_close(worst, TOL_1, f"config3 {variant}")


def test_batched_matches_single(gpu_lib):
    import torch
    shapes = [(256, 192, 48), (300, 130, 20), (256, 192, 48), (128, 512, 64), (96, 96, 96)]
    cases = [Case(_wl(m, n, r, seed=40 + i), MatrixSpec(0, "W", 0, m, n, r))
             for i, (m, n, r) in enumerate(shapes)]
    for c in cases:
        c.load_grad(0)
    for variant in (ORTH, DION):
        a = [(c.X.clone(), c.G, c.R.clone(), c.V.clone()) for c in cases]
        b = [(c.X.clone(), c.G, c.R.clone(), c.V.clone()) for c in cases]
        gpu_lib.step_batched(a, 0.01, 0.95, variant)
        for t in b:
            gpu_lib.step(*t, 0.01, 0.95, variant)
        torch.cuda.synchronize()
        for (xa, _, ra, va), (xb, _, rb, vb) in zip(a, b):
            for u, w in ((xa, xb), (ra, rb), (va, vb)):
                assert rel_fro(u.double().cpu().numpy(), w.double().cpu().numpy()) < 1e-5


def test_plan_api_matches_step_batched(gpu_lib):
    import torch
    shapes = [(384, 256, 64), (256, 384, 32)]
    cases = [Case(_wl(m, n, r, "bf16", seed=60 + i), MatrixSpec(0, "W", 0, m, n, r))
             for i, (m, n, r) in enumerate(shapes)]
    for c in cases:
        c.load_grad(0)
    a = [(c.X.clone(), c.G, c.R.clone(), c.V.clone()) for c in cases]
    b = [(c.X.clone(), c.G, c.R.clone(), c.V.clone()) for c in cases]
    plan = gpu_lib.Plan(a, "orth")
    ws = plan.new_workspace()
    plan.step(0.01, 0.95, ws)
    assert gpu_lib.status(ws, plan.count)[0] == 0
    plan.close()
    gpu_lib.step_batched(b, 0.01, 0.95, "orth")
    torch.cuda.synchronize()
    for ta, tb in zip(a, b):
        for u, w in zip(ta, tb):
            assert torch.equal(u, w)


# Wide W (n >> m): Dion's column norms run in up to 64 row slices of W with a
# ragged last slice, over whole and partial 64-column groups.
@pytest.mark.parametrize("m,n,r", [(48, 33001, 24), (160, 9000, 130)])
@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_wide_right_factor(gpu_lib, m, n, r, variant, arith):
    wl = _wl(m, n, r, "bf16")
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    say(f"wide {m}x{n} r={r} {variant} {arith}")
    gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, variant, math=arith)
    res, x_prev = c.oracle(variant)
    assert_close(c.errors(x_prev, res.M), TOL_1, f"wide {m}x{n} r={r} {variant} {arith}")


# One grouped call over classes of 1, 3, 4 and 5 Cholesky blocks: the
# look-ahead pairs run for all classes together, and each class's block
# steps stop at its own last block.
@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_batched_mixed_block_counts(gpu_lib, variant, arith):
    shapes = [(400, 300, 150), (256, 192, 48), (700, 650, 300), (300, 260, 250)]
    cases = [Case(_wl(m, n, r, "bf16", seed=80 + i), MatrixSpec(0, "W", 0, m, n, r))
             for i, (m, n, r) in enumerate(shapes)]
    for c in cases:
        c.load_grad(0)
    say(f"mixed block counts {variant} {arith}")
    gpu_lib.step_batched([(c.X, c.G, c.R, c.V) for c in cases], 0.01, 0.95, variant, math=arith)
    for c, (m, n, r) in zip(cases, shapes):
        res, x_prev = c.oracle(variant)
        assert_close(c.errors(x_prev, res.M), TOL_1, f"mixed {m}x{n} r={r} {variant} {arith}")


# The same classes six times over (306 blocks of T and Y: more than the
# one-launch factorization takes, so the launch-per-step chain runs): every
# copy of a matrix has the inputs of the first, whose step is checked
# against the oracle, and must come out bitwise equal to it.
@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_batched_mixed_block_counts_chain(gpu_lib, variant, arith):
    import torch
    shapes = [(400, 300, 150), (256, 192, 48), (700, 650, 300), (300, 260, 250)]
    blocks = sum((r + 63) // 64 * ((r + 63) // 64) for _, _, r in shapes)
    copies = 6
    assert copies * blocks > 256
    cases = [Case(_wl(m, n, r, "bf16", seed=80 + i), MatrixSpec(0, "W", 0, m, n, r))
             for i, (m, n, r) in enumerate(shapes)]
    for c in cases:
        c.load_grad(0)
    extra = [[(c.X.clone(), c.G, c.R.clone(), c.V.clone()) for c in cases] for _ in range(copies - 1)]
    say(f"mixed block counts, chain {variant} {arith}")
    mats = [(c.X, c.G, c.R, c.V) for c in cases] + [t for e in extra for t in e]
    ws = gpu_lib.step_batched(mats, 0.01, 0.95, variant, math=arith)
    assert gpu_lib.status(ws, len(mats))[0] == 0
    torch.cuda.synchronize()
    for c, (m, n, r) in zip(cases, shapes):
        res, x_prev = c.oracle(variant)
        assert_close(c.errors(x_prev, res.M), TOL_1, f"mixed chain {m}x{n} r={r} {variant} {arith}")
    for e in extra:
        for c, (x, _, rr, v) in zip(cases, e):
            assert torch.equal(x, c.X) and torch.equal(rr, c.R) and torch.equal(v, c.V)
