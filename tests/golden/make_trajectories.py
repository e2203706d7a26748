"""Writes the float64 oracle's long-horizon trajectories that the GPU tests
compare libdion with (tests/test_gpu_horizon.py).

    python tests/golden/make_trajectories.py [job ...]

Calls only oracle/ (run_steps) and the seeded input streams of workloads/.
For each job (a workload, a sample of its matrices, a step count and the
horizons to record) and each sampled matrix and rule, it runs the step from
the workload's initial state over the seeded gradients G_0, G_1, ... twice:
in float64 throughout, and with X, R, V rounded to float32 after every step
(run_steps(state_rounding="fp32"), the divergence that rounding the state
alone produces: the float32-state floor).  At every horizon it stores, per
matrix and rule, for the float64 trajectory:

  norms   Frobenius norms of X, R, V and dX = X - X_0
  samples the entries of X, R, V and dX at fixed seeded positions
  floor   relative Frobenius distance of the float32-state trajectory from
          the float64 one, for X, R, V and dX

into tests/golden/trajectory_<job>.npz (one array per quantity, keys
"<matrix>/<rule>/<horizon>/<name>", plus the sample positions "<matrix>/
pos_mn" and "<matrix>/pos_nr").  The relative error of a GPU result b
against the float64 a is then estimated as

  sqrt(N / k * sum over the k samples of (b - a)^2) / ||a||_F

(N entries in all), which for k = 512 random positions is within a few
percent of the exact value for errors spread over the matrix.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import run_steps  # noqa: E402
from oracle.checks import rel_fro  # noqa: E402
from workloads import MatrixStream, config  # noqa: E402

SAMPLES = 512

# name: (workload, matrix indices, steps, horizons, rules)
JOBS = {
    # the planted 2048 x 2048 matrix at rank 512 (its float32-state floor is
    # a diagnostic of the live, re-seeded test)
    "planted2048": (lambda: config(2), (0,), 100, (1, 10, 20, 50, 100), ("orth", "dion")),
    # 160M stack: one matrix of each shape class, first and last layer
    "gpt160m": (lambda: config(3), (0, 4, 5, 66, 70, 71), 100, (1, 10, 100), ("orth", "dion")),
    # 3B stack at rank 1/4: one matrix of each shape class of layer 0
    # (Q 3072x3072, K 3072x1024, gate 3072x8192, down 8192x3072)
    "llama3b_r4": (lambda: config(4, 4), (0, 1, 4, 6), 100, (1, 10, 100), ("orth", "dion")),
    # the 70B-style MLP up-projection at rank 512
    "mlp70b_r512": (lambda: config(5, r=512), (0,), 20, (1, 5, 20), ("orth", "dion")),
}


def positions(seed: int, total: int, k: int) -> np.ndarray:
    g = np.random.default_rng([seed, 7, 7])
    return np.sort(g.choice(total, size=min(k, total), replace=False)).astype(np.int64)


def run_job(name: str) -> str:
    make_wl, indices, steps, horizons, rules = JOBS[name]
    wl = make_wl()
    out = {}
    eta, beta = float(np.float32(wl.eta)), float(np.float32(wl.beta))
    for idx in indices:
        spec = wl.mats[idx]
        st = MatrixStream(wl, spec)
        x0, r0, v0 = (a.astype(np.float64) for a in st.init())
        pos_mn = positions(idx, spec.m * spec.n, SAMPLES)
        pos_nr = positions(idx + 1000, spec.n * spec.r, SAMPLES)
        out[f"{idx}/pos_mn"] = pos_mn
        out[f"{idx}/pos_nr"] = pos_nr
        for rule in rules:
            t0 = time.time()
            exact = (x0, r0, v0)
            rounded = (x0, r0, v0)
            done = 0
            for h in horizons:
                grads = [st.grad_f64(t) for t in range(done, h)]
                exact = run_steps(*exact, grads, eta, beta, rule)
                rounded = run_steps(*rounded, grads, eta, beta, rule, state_rounding="fp32")
                del grads
                done = h
                X, R, V = exact
                dX = X - x0
                key = f"{idx}/{rule}/{h}"
                out[key + "/norms"] = np.array([np.linalg.norm(X), np.linalg.norm(R),
                                                np.linalg.norm(V), np.linalg.norm(dX)])
                out[key + "/X"] = X.ravel()[pos_mn]
                out[key + "/R"] = R.ravel()[pos_mn]
                out[key + "/dX"] = dX.ravel()[pos_mn]
                out[key + "/V"] = V.ravel()[pos_nr]
                Xf, Rf, Vf = rounded
                out[key + "/floor"] = np.array([rel_fro(Xf, X), rel_fro(Rf, R), rel_fro(Vf, V),
                                                rel_fro(Xf - x0, dX)])
                print(f"{name} matrix {idx} ({spec.m}x{spec.n} r={spec.r}) {rule} step {h}: "
                      f"floor X R V dX {out[key + '/floor']}  ({time.time() - t0:.0f} s)",
                      flush=True)
            del exact, rounded
    path = os.path.join(HERE, f"trajectory_{name}.npz")
    np.savez_compressed(path, **out)
    return path


def main(argv) -> int:
    names = argv or list(JOBS)
    for name in names:
        print("wrote", run_job(name), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
