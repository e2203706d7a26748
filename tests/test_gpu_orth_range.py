"""orth() over the whole range of conditioning (GPU).

The symbol list of the Orth-Dion page defines orth as the QR
orthonormalization of the column space; with a positive diagonal it is the
Q factor, for any full-rank factor.  These tests take factors P = M V or
W = M^T U with nearly collinear columns and condition numbers of about 1e4
and 1e6 (planted spectra, workloads.conditioned_inputs, side "P" or "W"),
where one CholeskyQR pass is not enough, and check every stage of libdion's
step against the oracle's definition applied to the library's own float32
inputs to that stage (read back with dion_plan_buffer):

  P  = M V              against M V in float64
  U  = orth(P)          against the oracle's qr_pos(P) (Householder, float64)
  W  = M^T U            against M^T U in float64
  Vbar                  against qr_pos(W) (Orth-Dion) or colnorm(W) (Dion)
  X, R                  against X - eta U Vbar^T and beta (M - U W^T)

orth is checked at 1e-5 relative: a two-pass orth reproduces the Q factor
of its float32 input to about float32 rounding however ill-conditioned the
input is.  A product C = A B is checked by the bound that holds for any
summation order, |C - AB| against |A| |B| (relative Frobenius), at its
arithmetic's accuracy.  The whole step is not compared with the oracle's
step on the original inputs here: at these condition numbers the float32
product M V alone moves the Q factor by about kappa times float32's
rounding, for any float32 implementation, so each stage is compared on the
library's own inputs to it instead."""
import numpy as np
import pytest

from oracle import Breakdown, colnorm, qr_pos
from workloads import bf16_bits_to_f32, conditioned_inputs

from .gpuhelp import f32, say

pytestmark = pytest.mark.gpu

ETA, BETA = 0.01, 0.95
# relative accuracy of one m x n x r product: float32 products (2^-24 per
# term, summed) and split-bfloat16 products (up to 2^-16 per term)
PROD_TOL = {"f32": 1e-5, "bf16x3": 2e-4}
ORTH_TOL = 1e-5
CTL_TWO, CTL_RETRY = 1 << 8, 1 << 9


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _run(gpu_lib, cases, variant, arith):
    """Grouped step through a plan over `cases` (lists of numpy inputs);
    returns per matrix the device outputs and the intermediate factors."""
    import torch
    mats = []
    for X, G, R, V in cases:
        Gd = (torch.from_numpy(G.view(np.int16)).view(torch.bfloat16) if G.dtype == np.uint16
              else torch.from_numpy(G)).cuda()
        mats.append(tuple(t.cuda() if not t.is_cuda else t for t in
                          (torch.from_numpy(X.copy()), Gd, torch.from_numpy(R.copy()),
                           torch.from_numpy(V.copy()))))
    plan = gpu_lib.Plan(mats, variant, math=arith)
    ws = plan.new_workspace()
    plan.step(ETA, BETA, ws)
    rc, per = gpu_lib.status(ws, plan.count)
    raw = ws[:4 * plan.count].view(torch.int32).cpu().numpy().copy()
    out = []
    for i, (X, G, R, V) in enumerate(mats):
        out.append({k: t.double().cpu().numpy() for k, t in
                    (("X", X), ("R", R), ("V", V), ("P", plan.buffer(ws, gpu_lib.BUF_P, i)),
                     ("U", plan.buffer(ws, gpu_lib.BUF_U, i)),
                     ("W", plan.buffer(ws, gpu_lib.BUF_W, i)))})
    plan.close()
    return rc, per, raw, out


def _prod_err(c, a, b):
    """|c - a b|_F / | |a| |b| |_F."""
    return float(np.linalg.norm(c - a @ b) / np.linalg.norm(np.abs(a) @ np.abs(b)))


def _check_stages(case, o, variant, arith, what):
    X0, G, R0, V0 = (a.astype(np.float64) if a.dtype != np.uint16 else
                     bf16_bits_to_f32(a).astype(np.float64) for a in case)
    eta, beta = f32(ETA), f32(BETA)
    M = G + R0
    r = V0.shape[1]
    dx = o["X"] - X0
    # X is stored in float32: its rounding (2^-24 |X|) adds to the update's
    ux = 2.0 ** -24 * np.linalg.norm(o["X"])
    err = {
        "P": _prod_err(o["P"], M, V0),
        "U": _rel(o["U"], qr_pos(o["P"])[0]),
        "W": _prod_err(o["W"], M.T, o["U"]),
        "V": _rel(o["V"], qr_pos(o["W"])[0] if variant == "orth" else colnorm(o["W"])),
        "dX": float(np.linalg.norm(dx + eta * o["U"] @ o["V"].T) /
                    (eta * np.linalg.norm(np.abs(o["U"]) @ np.abs(o["V"]).T) + ux)),
        "R": float(np.linalg.norm(o["R"] - beta * (M - o["U"] @ o["W"].T)) /
                   (beta * (np.linalg.norm(M) + np.linalg.norm(np.abs(o["U"]) @ np.abs(o["W"]).T)))),
    }
    orth_u = np.abs(o["U"].T @ o["U"] - np.eye(r)).max()
    say(f"{what}: stage errors {err}, |U^T U - I| {orth_u:.1e}")
    tol = PROD_TOL[arith]
    for k in ("P", "W", "dX", "R"):
        assert err[k] <= tol, (what, k, err)
    for k in ("U", "V"):
        assert err[k] <= ORTH_TOL, (what, k, err)
    assert orth_u <= ORTH_TOL, (what, orth_u)
    if variant == "orth":
        assert np.abs(o["V"].T @ o["V"] - np.eye(r)).max() <= ORTH_TOL


@pytest.mark.parametrize("kappa", [1e4, 1e6])
@pytest.mark.parametrize("side", ["P", "W"])
@pytest.mark.parametrize("variant", ["orth", "dion"])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
@pytest.mark.parametrize("m,n,r,g_dtype", [(300, 200, 40, "f32"), (700, 520, 96, "bf16")])
def test_ill_conditioned_factors(gpu_lib, kappa, side, variant, arith, m, n, r, g_dtype):
    case = conditioned_inputs(m, n, r, kappa, seed=int(m + r + np.log10(kappa)),
                              g_dtype=g_dtype, side=side)
    what = f"{m}x{n} r={r} kappa={kappa:.0e} ({side}) {variant} {arith} {g_dtype}"
    say(what)
    rc, per, raw, out = _run(gpu_lib, [case], variant, arith)
    assert rc == 0, (what, per)
    # the control bits left are those of the last factorization: W's for
    # Orth-Dion, P's for Dion; the ill-conditioned one took two passes
    last_is_ill = (side == "W") == (variant == "orth")
    if last_is_ill:
        assert raw[0] & CTL_TWO, (what, hex(raw[0]))
        # beyond what a second pass repairs, the shifted first pass runs (a
        # bfloat16 G, or split-bfloat16 products, add rounding that lowers
        # the factor's condition number into the two-pass range)
        if kappa >= 1e6 and arith == "f32" and g_dtype == "f32":
            assert raw[0] & CTL_RETRY, (what, hex(raw[0]))
    _check_stages(case, out[0], variant, arith, what)


@pytest.mark.parametrize("variant", ["orth", "dion"])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_grouped_call_mixes_one_and_two_passes(gpu_lib, variant, arith):
    # each matrix takes its own number of passes inside the same launches;
    # the ill-conditioned side is the last factorization of the variant
    side = "W" if variant == "orth" else "P"
    cases = [conditioned_inputs(300, 200, 40, 1e6, seed=11, side=side),
             conditioned_inputs(256, 192, 48, 3.0, seed=12, side=side),
             conditioned_inputs(400, 300, 150, 1e4, seed=13, side=side),
             conditioned_inputs(200, 260, 20, 10.0, seed=14, side=side)]
    say(f"grouped mixed conditioning {variant} {arith}")
    rc, per, raw, out = _run(gpu_lib, cases, variant, arith)
    assert rc == 0, per
    assert raw[0] & CTL_TWO and raw[2] & CTL_TWO, [hex(v) for v in raw]
    assert not raw[1] & CTL_TWO and not raw[3] & CTL_TWO, [hex(v) for v in raw]
    for i, (case, o) in enumerate(zip(cases, out)):
        _check_stages(case, o, variant, arith, f"grouped matrix {i} {variant} {arith}")


@pytest.mark.parametrize("variant", ["orth", "dion"])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_exactly_dependent_columns_break_down(gpu_lib, variant, arith):
    # V0 with two equal columns: P = M V0 has two equal columns, which the
    # oracle's orth rejects; the library reports a breakdown of orth(P) and
    # leaves X, R, V as they were
    import torch
    X, G, R, V = conditioned_inputs(300, 200, 40, 10.0, seed=21, duplicate=6)
    with pytest.raises(Breakdown):
        qr_pos(G.astype(np.float64) @ V.astype(np.float64))
    Xd, Gd, Rd, Vd = (torch.from_numpy(a.copy()).cuda() for a in (X, G, R, V))
    ws = gpu_lib.step(Xd, Gd, Rd, Vd, ETA, BETA, variant, math=arith)
    rc, per = gpu_lib.status(ws, 1)
    assert rc == gpu_lib.ERR_BREAKDOWN and per[0] & gpu_lib.STATUS_ORTH_P, per
    for dev, host in ((Xd, X), (Rd, R), (Vd, V)):
        assert np.array_equal(dev.cpu().numpy(), host)


@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_two_pass_is_deterministic(gpu_lib, arith):
    for side in ("P", "W"):
        case = conditioned_inputs(300, 200, 40, 1e6, seed=31, side=side)
        a = _run(gpu_lib, [case], "orth", arith)[3][0]
        b = _run(gpu_lib, [case], "orth", arith)[3][0]
        for k in ("X", "R", "V", "U", "W"):
            assert np.array_equal(a[k], b[k]), (side, k)


@pytest.mark.parametrize("variant", ["orth", "dion"])
@pytest.mark.parametrize("arith", ["f32", "bf16x3"])
def test_ill_conditioned_many_matrices(gpu_lib, variant, arith):
    # 30 matrices at r = 150 (three 64-blocks a side, 270 blocks of T and
    # Y in the plan: more than one launch holds at once), mixing well- and
    # ill-conditioned factors on both sides, in one grouped step: the first
    # pass, its shifted retry and the second pass of every matrix must each
    # give the Q factor of the library's own input
    m, n, r = 300, 260, 150
    cases, names = [], []
    for i in range(30):
        kappa = (10.0, 1e4, 1e6)[i % 3]
        side = "P" if (i // 3) % 2 == 0 else "W"
        cases.append(conditioned_inputs(m, n, r, kappa, seed=500 + i, g_dtype="f32", side=side))
        names.append(f"matrix {i} kappa={kappa:.0e} ({side})")
    say(f"30 matrices {m}x{n} r={r} {variant} {arith}")
    rc, per, raw, out = _run(gpu_lib, cases, variant, arith)
    assert rc == 0, per
    for case, o, what in zip(cases, out, names):
        _check_stages(case, o, variant, arith, f"{what} {variant} {arith}")
