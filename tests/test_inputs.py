"""The seeded input generators: determinism, addressability, rounding, shapes."""
import numpy as np
import pytest
import torch

from workloads import (CONFIGS, MatrixStream, bf16_bits_to_f32, config,
                       f32_to_bf16_bits)


def test_streams_are_deterministic_and_addressable():
    wl = config(1)
    a = MatrixStream(wl, wl.mats[0])
    b = MatrixStream(wl, wl.mats[0])
    x0a, r0a, v0a = a.init()
    x0b, _, v0b = b.init()
    assert np.array_equal(x0a, x0b) and np.array_equal(v0a, v0b)
    assert not r0a.any()
    # step 5 drawn directly equals step 5 drawn after steps 0..4
    direct = MatrixStream(wl, wl.mats[0]).grad(5)
    for t in range(5):
        a.grad(t)
    assert np.array_equal(a.grad(5), direct)
    assert not np.array_equal(a.grad(4), direct)


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * 3.0,
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3.4e38,
                  -3.4e38, 1e-40, np.inf, -np.inf], dtype=np.float32),
    ])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = bf16_bits_to_f32(ours)
    ref_back = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(back, ref_back)
    nan = f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(bf16_bits_to_f32(nan)[0])


@pytest.mark.parametrize("key", [1, 2])
def test_init_state_recipe(key):
    wl = CONFIGS[key]()
    s = MatrixStream(wl, wl.mats[0])
    x0, r0, v0 = s.init()
    spec = wl.mats[0]
    assert x0.shape == (spec.m, spec.n) and x0.dtype == np.float32
    assert v0.shape == (spec.n, spec.r) and v0.dtype == np.float32
    v = v0.astype(np.float64)
    assert np.max(np.abs(v.T @ v - np.eye(spec.r))) < 1e-6
    assert abs(np.std(x0) - 0.02) < 0.002


def test_config_shapes():
    c3 = config(3)
    assert c3.count == 72 and c3.elements == 84_934_656
    assert {(s.m, s.n, s.r) for s in c3.mats} == {(768, 768, 192), (768, 3072, 192),
                                                  (3072, 768, 192)}
    c4 = config(4, 4)
    assert c4.count == 196 and c4.elements == 2_818_572_288
    assert {(s.m, s.n, s.r) for s in c4.mats} == {
        (3072, 3072, 768), (3072, 1024, 256), (3072, 8192, 768), (8192, 3072, 768)}
    c16 = config(4, 16)
    assert {(s.m, s.n, s.r) for s in c16.mats} == {
        (3072, 3072, 192), (3072, 1024, 64), (3072, 8192, 192), (8192, 3072, 192)}
    assert c4.g_dtype == "bf16" and config(3).g_dtype == "f32"
    c5 = config(5, r=2048)
    assert (c5.mats[0].m, c5.mats[0].n, c5.mats[0].r) == (8192, 28672, 2048)


def test_planted_gradient_spectrum():
    # A small planted stream: the leading singular values are 1/k plus noise.
    from workloads.configs import MatrixSpec, Workload
    wl = Workload(name="t", seed=9, mats=(MatrixSpec(0, "W", 0, 200, 150, 10),),
                  g_dtype="f32", g_kind="planted", noise=(1e-4,), planted_rank=8,
                  eta=0.01, beta=0.95, steps=1, variants=("orth",))
    s = MatrixStream(wl, wl.mats[0])
    sv = np.linalg.svd(s.grad(0).astype(np.float64), compute_uv=False)
    np.testing.assert_allclose(sv[:8], 1.0 / np.arange(1, 9), rtol=5e-3)
    assert sv[8] < 0.01
