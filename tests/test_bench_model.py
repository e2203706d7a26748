"""bench.py's roofline arithmetic (CPU).

The step roofline is T_roof = max(B_min / 8.0 TB/s, F_alg / P_used) with
B_min = (16 + e_G) m n + 8 n r bytes (read X, G, R, V; write X, R, V) and
F_alg = 8 m n r + 4 m r^2 + (4 n r^2 for Orth-Dion, 3 n r for Dion), P_used
the float32 matrix peak (157.3 TFLOP/s) or a third of the bfloat16 peak
(2516.6 TFLOP/s) for split-bfloat16 products.  The figures below were worked
out by hand from each workload's shapes before the benchmark existed; the
test checks that the code the benchmark reports with gives them back.
"""
import math

import pytest

import bench
from workloads import config

# workload, variant, e_G, B_min (GB), F_alg (TFLOP), T_roof float32 (ms),
# T_roof split-bfloat16 (ms)
FIGURES = [
    ((2,), "orth", 4, 0.0923, 0.0215, 0.1365, 0.0256),
    ((2,), "dion", 4, 0.0923, 0.0193, 0.1229, 0.0230),
    ((3,), "orth", 4, 1.826, 0.1549, 0.985, 0.228),
    ((3,), "dion", 4, 1.826, 0.1427, 0.907, 0.228),
    ((4, 4), "orth", 2, 55.26, 19.70, 125.2, 23.5),
    ((4, 4), "dion", 2, 55.26, 18.00, 114.4, 21.5),
    ((4, 16), "orth", 2, 51.86, 4.343, 27.6, 6.48),
    ((4, 16), "dion", 2, 51.86, 4.237, 26.9, 6.48),
    ((5, None, 512), "orth", 2, 4.345, 1.001, 6.36, 1.19),
    ((5, None, 2048), "orth", 2, 4.698, 4.467, 28.4, 5.32),
]


def _shapes(key):
    if len(key) == 3:
        wl = config(key[0], r=key[2])
    else:
        wl = config(*key)
    return [(s.m, s.n, s.r) for s in wl.mats]


@pytest.mark.parametrize("key,variant,eg,bmin_gb,f_tflop,t32_ms,t3_ms", FIGURES)
def test_step_roofline_figures(key, variant, eg, bmin_gb, f_tflop, t32_ms, t3_ms):
    shapes = _shapes(key)
    flops, bmin = bench.step_model(shapes, variant, eg)
    assert math.isclose(bmin / 1e9, bmin_gb, rel_tol=2e-3), bmin
    assert math.isclose(flops / 1e12, f_tflop, rel_tol=3e-3), flops
    t32, _, _, _ = bench.step_roofline(shapes, variant, eg, "f32")
    t3, _, _, _ = bench.step_roofline(shapes, variant, eg, "bf16x3")
    assert math.isclose(t32 * 1e3, t32_ms, rel_tol=3e-3), t32
    assert math.isclose(t3 * 1e3, t3_ms, rel_tol=5e-3), t3


def test_step_roofline_entry_fraction():
    # the reported fraction is T_roof / T_measured, and the bound names the
    # larger of the two times
    shapes = _shapes((4, 4))
    t_roof, t_mfma, flops, bmin = bench.step_roofline(shapes, "orth", 2, "bf16x3")
    e = bench.step_roofline_entry(shapes, "orth", 2, "bf16x3", 2 * t_roof)
    assert e["bound"] == "mfma" and math.isclose(e["frac"], 0.5, abs_tol=1e-4)
    assert math.isclose(e["p_used_tflops"], 2516.6 / 3, rel_tol=1e-3)
    shapes16 = _shapes((4, 16))
    e16 = bench.step_roofline_entry(shapes16, "orth", 2, "bf16x3", 0.010)
    assert e16["bound"] == "hbm"
    assert math.isclose(e16["effective_gbps"], 51.86 / 0.010, rel_tol=2e-3)


def test_phase_model_sums_to_the_step():
    # the five phases' algorithmic flops add up to the step's, plus the
    # (4/3) r^3 of each Cholesky factorization that the phases charge to
    # orth (one per matrix for Dion, two for Orth-Dion)
    for key, variant, eg in (((4, 4), "orth", 2), ((3,), "dion", 4)):
        shapes = _shapes(key)
        f, _ = bench.phase_model(shapes, variant, eg)
        flops, _ = bench.step_model(shapes, variant, eg)
        chol = sum(4.0 / 3.0 * r ** 3 for (_, _, r) in shapes) * (2 if variant == "orth" else 1)
        assert math.isclose(sum(f.values()), flops + chol, rel_tol=1e-12)
