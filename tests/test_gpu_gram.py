"""The sliced int8 Gram matrix against the float64 MFMA Gram matrix (GPU).

Stage 0 of a single-shard DION_SHARDED plan leaves P^T P (P = M V) in its
Gram exchange buffer.  Two plans that differ only in DION_GRAM_F64 compute
the same P with the same kernels, so their buffers differ by the Gram
arithmetic alone: float32 products summed in float64 (products exact), or
five base-128 digits per column scaled by a power of two, with the 15
leading digit products summed exactly in int32.  The digit form truncates
each entry of a column below 2^-35 of the column's largest entry, so each
Gram entry should agree to about 1e-11 of sqrt(S_ii S_jj); the bound here
is 1e-9.  Cases cover ragged row and column counts, a row count past the
int32 flush interval of the int8 kernel (65,536 rows), columns of widely
different scale and an all-zero column.
"""
import numpy as np
import pytest

from workloads.configs import MatrixSpec, Workload

from .gpuhelp import Case, say

pytestmark = pytest.mark.gpu

GRAM_TOL = 1e-9


def _case(m, n, r, seed, g_dtype="f32"):
    wl = Workload(name="gram", seed=seed, mats=(MatrixSpec(0, "W", 0, m, n, r),),
                  g_dtype=g_dtype, g_kind="normal", noise=(1.0,), planted_rank=0, eta=0.01,
                  beta=0.95, steps=1, variants=("orth",))
    c = Case(wl, wl.mats[0])
    c.load_grad(0)
    return c


def _gram(gpu_lib, c, math, v_scale=None):
    """P^T P from stage 0 of a one-shard plan (upper triangle, float64)."""
    import torch
    V = c.V.clone()
    if v_scale is not None:
        V *= torch.as_tensor(v_scale, dtype=V.dtype, device=V.device)
    plan = gpu_lib.Plan([(c.X.clone(), c.G.clone(), c.R.clone(), V)], "orth", math=math, sharded=True)
    ws = plan.new_workspace()
    plan.shard_stage(0, 0.01, 0.95, ws)
    torch.cuda.synchronize()
    S = plan.shard_buffer(ws, gpu_lib.SHARD_GRAM, 0).cpu().numpy().copy()
    plan.close()
    r = c.V.shape[1]
    return np.triu(S[:r, :r])


def _compare(gpu_lib, c, arith, v_scale=None):
    base = gpu_lib.MATH[arith]
    s8 = _gram(gpu_lib, c, base, v_scale)
    s64 = _gram(gpu_lib, c, base | gpu_lib.GRAM_F64, v_scale)
    d = np.sqrt(np.abs(np.diag(s64)))
    norm = np.outer(d, d)
    norm[norm == 0] = 1.0
    err = np.abs(s8 - s64) / norm
    say(f"  max normwise entry difference {err.max():.3e}")
    assert np.all(np.isfinite(s8))
    assert err.max() <= GRAM_TOL, err.max()
    return s8, s64


@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
@pytest.mark.parametrize("m,n,r", [
    (700, 300, 40),      # one ragged 64-wide tile, ragged rows
    (1536, 512, 256),    # 4 x 4 tiles, several reduction splits
    (333, 900, 130),     # ragged column block past two tiles
    (20, 96, 16),        # fewer rows than one 32-row block
])
def test_sliced_gram_matches_f64(gpu_lib, m, n, r, arith):
    say(f"gram {m}x{n} r={r} {arith}")
    _compare(gpu_lib, _case(m, n, r, seed=5), arith)


def test_sliced_gram_past_flush_interval(gpu_lib):
    # 70,000 rows in one reduction slice: the int32 level sums are moved to
    # float64 after 65,536 rows and once more at the end
    say("gram 70000x64 r=32")
    _compare(gpu_lib, _case(70000, 64, 32, seed=6), "bf16x3")


def test_sliced_gram_column_scales(gpu_lib):
    # columns of P scaled from 1e-30 to 1e30 and one column of zeros: each
    # column has its own power-of-two scale, so the normwise error is the
    # same for all of them
    m, n, r = 900, 400, 48
    c = _case(m, n, r, seed=7)
    scale = np.float32(10.0) ** np.linspace(-30, 30, r).astype(np.float32)
    scale[5] = 0.0
    say(f"gram {m}x{n} r={r} column scales 1e-30..1e30")
    s8, s64 = _compare(gpu_lib, c, "f32", v_scale=scale)
    assert np.all(s8[5, :] == 0.0) and np.all(s8[:, 5] == 0.0)


@pytest.mark.parametrize("m", [16384, 16640])
def test_sliced_gram_fused_maxima_boundary(gpu_lib, m):
    # P = M V on the 256 x 256 split-bfloat16 tiles without a reduction
    # split: at most 64 row tiles (16,384 rows) leave their column maxima
    # for the Gram matrix; 65 row tiles fall back to the column-maximum pass
    say(f"gram {m}x256 r=256 bf16x3 (row tiles {m // 256 + (m % 256 > 0)})")
    _compare(gpu_lib, _case(m, 256, 256, seed=8), "bf16x3")
