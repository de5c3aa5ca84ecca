"""Host-side checks of the seeded input generators (no GPU)."""

import numpy as np
import torch

import workloads


def test_shapes_and_determinism():
    d1 = workloads.make("c1")
    d2 = workloads.make("c1")
    assert d1["X"].shape == (1024, 16) and d1["Y"].shape == (1024, 16)
    assert d1["X"].dtype == np.float32
    np.testing.assert_array_equal(d1["X"], d2["X"])
    np.testing.assert_array_equal(d1["Y"], d2["Y"])
    assert not np.array_equal(d1["X"], d1["Y"][:, :16])
    np.testing.assert_allclose(d1["a"].sum(), 1.0, rtol=1e-6)


def test_resized_draws_keep_distribution_parameters():
    small = workloads.make("c5", n=300, m=77, d=40)
    w = small["w"]
    assert (w.n, w.m, w.d, w.eps, w.iters) == (300, 77, 40, 0.01, 300)
    assert small["V"].shape == (77, 128) and small["U"].shape == (300, 128)
    assert np.all(np.abs(small["Y"]) <= 1.0 / np.sqrt(40) + 1e-7)   # Uniform[-1,1]^d / sqrt(d)
    np.testing.assert_allclose(small["b"].sum(), 1.0, rtol=1e-6)
    assert np.all(small["a"] > 0)


def test_bf16_round_matches_torch_rne():
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]   # ties to even
    ours = workloads.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_bf16_workload_values_are_representable():
    d = workloads.make("c4", n=500, m=400)
    for k in ("X", "Y", "V"):
        v = d[k]
        np.testing.assert_array_equal(v, workloads.bf16_round(v))
