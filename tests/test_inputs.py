"""Checks of the seeded input generators (shared by oracle tests and GPU tests)."""
import numpy as np
import torch

from moe_inputs import (WORKLOADS, balanced_routing, bf16_round, expert_weight,
                        f32_to_bf16_bits, make_inputs, zipf_routing)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 3.0e38], np.float32)])
    ref = torch.tensor(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(a), ref)
    np.testing.assert_array_equal(bf16_round(bf16_round(a)), bf16_round(a))


def test_zipf_routing_properties():
    idx, g = zipf_routing(4096, 32, 4, 1.2, seed=0)
    assert idx.shape == (4096, 4) and idx.dtype == np.int32
    assert all(len(set(r)) == 4 for r in idx.tolist())
    c = np.bincount(idx.ravel(), minlength=32)
    assert c.sum() == 4096 * 4 and c[0] == c.max()  # rank 1 is the most popular
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=1e-6)
    assert (g > 0).all()


def test_zipf_zero_popularity_experts_never_chosen():
    pop = np.ones(16); pop[[2, 7]] = 0
    idx, _ = zipf_routing(512, 16, 4, 1.2, seed=1, popularity=pop)
    c = np.bincount(idx.ravel(), minlength=16)
    assert c[2] == 0 and c[7] == 0 and c.sum() == 2048


def test_balanced_routing_exact_counts():
    idx, g = balanced_routing(1024, 128, 4, seed=0)
    assert (np.bincount(idx.ravel(), minlength=128) == 32).all()
    assert all(len(set(r)) == 4 for r in idx.tolist())


def test_reproducible_and_streams_independent():
    wl = WORKLOADS["tiny_f32"]
    a, b = make_inputs(wl, 0), make_inputs(wl, 0)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])
    c = make_inputs(wl, 1)
    assert not np.array_equal(a["x"], c["x"])
    np.testing.assert_array_equal(a["w_up"][3], expert_weight(wl, "w_up", 3, 0))
    assert abs(a["w_gate"].std() - 0.02) < 0.002 and abs(a["x"].std() - 1) < 0.05


def test_bf16_workload_values_are_bf16():
    wl = WORKLOADS["bf16_e8"].with_shape(T=64, d=128, f=64)
    inp = make_inputs(wl, 0)
    for n in ("x", "dy", "w_router", "w_gate"):
        np.testing.assert_array_equal(bf16_round(inp[n]), inp[n])
