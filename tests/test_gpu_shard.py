"""Row-sharded (FSDP) step through the staged plan API (GPU).

One global matrix is cut into row shards X_i = X[a_i : a_i + m_i]; each
shard is a matrix of one DION_SHARDED plan with its own copy of V.  Between
the three stages the test sums the exchange buffers over the shards (what
an all-reduce across GPUs would do) and writes the sum back into every
shard's buffer.  The concatenated shards must then match the float64
oracle's step on the global matrix, to the one-step gate, and every shard
must hold the same Vbar.
"""
import numpy as np
import pytest

from oracle import DION, ORTH
from workloads.configs import MatrixSpec, Workload

from .gpuhelp import TOL_1, Case, f32, rel_fro, say

pytestmark = pytest.mark.gpu


def _global_case(m, n, r, g_dtype, seed):
    wl = Workload(name="shard", seed=seed, mats=(MatrixSpec(0, "W", 0, m, n, r),),
                  g_dtype=g_dtype, g_kind="normal", noise=(1.0,), planted_rank=0, eta=0.01,
                  beta=0.95, steps=1, variants=("orth", "dion"))
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    return wl, c


def _sharded_step(gpu_lib, c, bounds, variant, arith, eta, beta):
    """Run the staged step on the row shards [bounds[i], bounds[i+1]) of the
    case's device state; returns the per-shard (X, R, V) tensors."""
    import torch
    shards = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        shards.append((c.X[a:b].clone(), c.G[a:b].clone(), c.R[a:b].clone(), c.V.clone()))
    plan = gpu_lib.Plan(shards, variant, math=arith, sharded=True)
    ws = plan.new_workspace()

    def all_reduce(which):
        bufs = [plan.shard_buffer(ws, which, i) for i in range(len(shards))]
        total = torch.stack([b.clone() for b in bufs]).sum(0)
        for b in bufs:
            b.copy_(total)

    plan.shard_stage(0, eta, beta, ws)
    all_reduce(gpu_lib.SHARD_GRAM)
    plan.shard_stage(1, eta, beta, ws)
    all_reduce(gpu_lib.SHARD_W)
    plan.shard_stage(2, eta, beta, ws)
    rc, per = gpu_lib.status(ws, plan.count)
    plan.close()
    assert rc == 0, per
    return shards


@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
@pytest.mark.parametrize("variant", [ORTH, DION])
@pytest.mark.parametrize("m,n,r,bounds,g_dtype", [
    (700, 300, 40, (0, 233, 466, 700), "f32"),       # three ragged shards
    (1536, 512, 256, (0, 768, 1536), "bf16"),        # shards on the large split-bfloat16 tiles
    (300, 200, 100, (0, 300), "bf16"),               # a single shard: no exchange needed
    (512, 300, 200, (0, 128, 256, 384, 512), "f32"),  # every shard has fewer rows than r
])
def test_sharded_step_matches_global_oracle(gpu_lib, m, n, r, bounds, g_dtype, variant, arith):
    wl, c = _global_case(m, n, r, g_dtype, seed=11)
    say(f"shard {m}x{n} r={r} shards={bounds} {variant} {arith}")
    shards = _sharded_step(gpu_lib, c, bounds, variant, arith, wl.eta, wl.beta)
    res, x_prev = c.oracle(variant)
    X = np.concatenate([s[0].double().cpu().numpy() for s in shards])
    R = np.concatenate([s[2].double().cpu().numpy() for s in shards])
    errs = {"X": rel_fro(X, res.X), "R": rel_fro(R, res.R),
            "dX": rel_fro(X - x_prev, res.X - x_prev)}
    for i, s in enumerate(shards):
        errs[f"V{i}"] = rel_fro(s[3].double().cpu().numpy(), res.V)
    say(f"  errors {errs}")
    for k, e in errs.items():
        assert e <= TOL_1, (k, e)
    # every shard computed the same Vbar from the same summed W
    for s in shards[1:]:
        assert bool((s[3] == shards[0][3]).all())


def test_shard_api_errors(gpu_lib):
    import torch
    wl, c = _global_case(128, 64, 8, "f32", seed=3)
    mats = [(c.X, c.G, c.R, c.V)]
    plain = gpu_lib.Plan(mats, "orth")
    ws = plain.new_workspace()
    with pytest.raises(gpu_lib.DionError):
        plain.shard_stage(0, 0.01, 0.95, ws)
    with pytest.raises(gpu_lib.DionError):
        plain.shard_buffer(ws, gpu_lib.SHARD_GRAM, 0)
    plain.close()
    sharded = gpu_lib.Plan(mats, "orth", sharded=True)
    ws = sharded.new_workspace()
    with pytest.raises(gpu_lib.DionError):
        sharded.shard_stage(3, 0.01, 0.95, ws)
    with pytest.raises(gpu_lib.DionError):
        sharded.shard_buffer(ws, 2, 0)
    with pytest.raises(gpu_lib.DionError):
        sharded.shard_buffer(ws, gpu_lib.SHARD_W, 1)
    # a sharded plan also runs as a whole step: one shard is the whole matrix
    x0 = c.X.clone()
    sharded.step(wl.eta, wl.beta, ws)
    torch.cuda.synchronize()
    assert gpu_lib.status(ws, 1)[0] == 0
    res, x_prev = c.oracle(ORTH)
    assert rel_fro(c.X.double().cpu().numpy(), res.X) <= TOL_1
    assert not torch.equal(x0, c.X)
    sharded.close()
    with pytest.raises(gpu_lib.DionError):
        gpu_lib.step(c.X, c.G, c.R, c.V, wl.eta, wl.beta, gpu_lib.VARIANTS["orth"] | gpu_lib.SHARDED)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("variant", [ORTH, DION])
def test_sharded_wide_tiles(gpu_lib, variant):
    # A 4096 x 16500 matrix at r = 152 in 16 row shards of 256: the shards'
    # M^T U launch has 16 x 65 = 1,040 tiles, enough for the 256 x 192
    # split-bfloat16 tiles, whose column maxima a sharded plan takes afresh
    # from the exchanged W.
    m, n, r = 4096, 16500, 152
    bounds = tuple(range(0, m + 1, 256))
    wl, c = _global_case(m, n, r, "bf16", seed=12)
    say(f"shard wide tiles {m}x{n} r={r} {len(bounds) - 1} shards {variant}")
    shards = _sharded_step(gpu_lib, c, bounds, variant, "bf16x3", wl.eta, wl.beta)
    res, x_prev = c.oracle(variant)
    X = np.concatenate([s[0].double().cpu().numpy() for s in shards])
    R = np.concatenate([s[2].double().cpu().numpy() for s in shards])
    errs = {"X": rel_fro(X, res.X), "R": rel_fro(R, res.R),
            "dX": rel_fro(X - x_prev, res.X - x_prev),
            "V": rel_fro(shards[0][3].double().cpu().numpy(), res.V)}
    say(f"  errors {errs}")
    for k, e in errs.items():
        assert e <= TOL_1, (k, e)
    for s in shards[1:]:
        assert bool((s[3] == shards[0][3]).all())
