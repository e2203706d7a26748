"""dion_step_noalloc, the entry point for callers that cannot allocate
device memory (GPU): it runs the same step as dion_step with the library's
own scratch, so on the same inputs the two give the same bits.  Two calls in
a row, the second on a smaller matrix, each checked against dion_step; the
status word it can copy out; shapes beyond its scratch are rejected before
any work."""
import numpy as np
import pytest

from workloads.configs import MatrixSpec, Workload

from .gpuhelp import Case, say

pytestmark = pytest.mark.gpu


def _case(m, n, r, g_dtype, seed):
    wl = Workload(name="noalloc", seed=seed, mats=(MatrixSpec(0, "W", 0, m, n, r),),
                  g_dtype=g_dtype, g_kind="normal", noise=(1.0,), planted_rank=0, eta=0.01,
                  beta=0.95, steps=1, variants=("orth", "dion"))
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    return c


@pytest.mark.parametrize("variant", ["orth", "dion"])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_noalloc_matches_step(gpu_lib, variant, arith):
    import torch
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    for (m, n, r, gd) in ((700, 520, 96, "bf16"), (256, 128, 16, "f32")):
        say(f"noalloc {m}x{n} r={r} {gd} {variant} {arith}")
        c = _case(m, n, r, gd, seed=m + r)
        a = [c.X.clone(), c.G, c.R.clone(), c.V.clone()]
        b = [c.X.clone(), c.G, c.R.clone(), c.V.clone()]
        gpu_lib.step_noalloc(*a, 0.01, 0.95, variant, status_out=status, math=arith)
        ws = gpu_lib.step(*b, 0.01, 0.95, variant, math=arith)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        assert int(status.item()) & 0xff == 0
        assert gpu_lib.status(ws, 1)[0] == 0
        # the oracle's step on the same inputs, at the one-step bar
        res, x_prev = c.oracle(variant)
        X = a[0].double().cpu().numpy()
        from oracle.checks import rel_fro
        err = {"X": rel_fro(X, res.X), "R": rel_fro(a[2].double().cpu().numpy(), res.R),
               "V": rel_fro(a[3].double().cpu().numpy(), res.V),
               "dX": rel_fro(X - x_prev, res.X - x_prev)}
        assert max(err.values()) <= 1e-4, err


def test_noalloc_reports_breakdown_and_rejects_large_shapes(gpu_lib):
    import torch
    c = _case(300, 200, 40, "f32", seed=3)
    c.G.zero_()
    before = [t.clone() for t in (c.X, c.R, c.V)]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_lib.step_noalloc(c.X, c.G, c.R, c.V, 0.01, 0.95, "orth", status_out=status)
    torch.cuda.synchronize()
    assert int(status.item()) & gpu_lib.STATUS_ORTH_P
    for x, y in zip(before, (c.X, c.R, c.V)):
        assert torch.equal(x, y)
    big = _case(2048, 2048, 512, "f32", seed=4)
    with pytest.raises(gpu_lib.DionError) as e:
        gpu_lib.step_noalloc(big.X, big.G, big.R, big.V, 0.01, 0.95, "orth")
    assert e.value.code == gpu_lib.ERR_WORKSPACE
    # a failed call leaves the next one working
    ok = _case(256, 128, 16, "f32", seed=5)
    ref = [ok.X.clone(), ok.G, ok.R.clone(), ok.V.clone()]
    gpu_lib.step_noalloc(ok.X, ok.G, ok.R, ok.V, 0.01, 0.95, "dion")
    gpu_lib.step(*ref, 0.01, 0.95, "dion")
    torch.cuda.synchronize()
    assert torch.equal(ok.X, ref[0]) and torch.equal(ok.V, ref[3])
    np.testing.assert_array_equal(ok.R.cpu().numpy(), ref[2].cpu().numpy())
