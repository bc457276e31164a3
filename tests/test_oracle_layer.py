"""Pins for the oracle's expert FFN, combine and whole-layer forward."""
import math

import numpy as np
import pytest
import torch

from moe_inputs import WORKLOADS, make_inputs
from oracle import moe_oracle as O


def tiny_inputs(T=24, d=8, E=4, k=2, f=6, seed=0, routing="learned", dtype="f32"):
    wl = WORKLOADS["tiny_f32"].with_shape(T=T, d=d, E=E, k=k, f=f, routing=routing, dtype=dtype)
    return wl, make_inputs(wl, seed)


def test_swiglu_worked_example():
    # One expert, d = f = 1. With x = 1 and W_gate = ln 3 the gate branch is
    # G = ln 3, whose logistic value is exactly 3/4; W_up = 2, W_down = -5.
    # H = G * 3/4 * 2 = 1.5 ln 3 and O = -7.5 ln 3.
    xp = np.array([[1.0]])
    G, U, H, Ov = O.ffn_forward(xp, np.array([[[math.log(3)]]]), np.array([[[2.0]]]),
                                np.array([[[-5.0]]]), np.array([0, 1]))
    assert abs(H[0, 0] - 1.5 * math.log(3)) < 1e-15
    assert abs(Ov[0, 0] + 7.5 * math.log(3)) < 1e-14
    # G = -ln 3 gives logistic 1/4; G = 0 gives H = 0 exactly.
    _, _, H2, _ = O.ffn_forward(np.array([[1.0], [0.0]]), np.array([[[-math.log(3)]]]),
                                np.array([[[1.0]]]), np.array([[[1.0]]]), np.array([0, 2]))
    assert abs(H2[0, 0] + 0.25 * math.log(3)) < 1e-15 and H2[1, 0] == 0.0


def test_single_expert_top1_is_dense_swiglu():
    # E = 1, k = 1: every gate is 1 and the layer is a dense SwiGLU FFN;
    # compared against torch's silu in fp64.
    wl, inp = tiny_inputs(T=30, d=8, E=1, k=1, f=12)
    out = O.layer_forward(inp, 1)
    x = torch.tensor(inp["x"], dtype=torch.float64)
    wg, wu, wd = (torch.tensor(inp[n][0], dtype=torch.float64) for n in ("w_gate", "w_up", "w_down"))
    ref = (torch.nn.functional.silu(x @ wg) * (x @ wu)) @ wd
    np.testing.assert_allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-15)


def test_identity_experts_return_input():
    # With the FFN replaced by the identity (O := Xp), dispatch followed by the
    # gate-weighted combine returns sum_j g_tj x_t = x_t.
    wl, inp = tiny_inputs(T=40, d=8, E=6, k=3)
    idx, g = O.route(O.router_logits(inp["x"], inp["w_router"]), 3)
    counts, offsets, rs, tr = O.dispatch_plan(idx, 6)
    xp = O.gather_rows(inp["x"], tr)
    np.testing.assert_allclose(O.combine(xp, g, rs), inp["x"], rtol=1e-14, atol=1e-15)


def test_layer_matches_per_token_loop():
    # Independent formulation: no dispatch at all; for each token apply its
    # k experts to its own row and sum with the gates.
    wl, inp = tiny_inputs(T=20, d=8, E=5, k=2, f=6)
    out = O.layer_forward(inp, 2)
    x = inp["x"].astype(np.float64)
    for t in range(20):
        acc = np.zeros(8)
        for j in range(2):
            e = out["topk_idx"][t, j]
            gt = x[t] @ inp["w_gate"][e].astype(np.float64)
            up = x[t] @ inp["w_up"][e].astype(np.float64)
            h = gt / (1 + np.exp(-gt)) * up
            acc += out["gates"][t, j] * (h @ inp["w_down"][e].astype(np.float64))
        np.testing.assert_allclose(out["y"][t], acc, rtol=1e-12, atol=1e-15)


def test_token_permutation_invariance():
    wl, inp = tiny_inputs(T=32, d=8, E=4, k=2, f=6, seed=3)
    out = O.layer_forward(inp, 2)
    bwd = O.layer_backward(inp, out)
    perm = np.random.default_rng(0).permutation(32)
    inp2 = dict(inp, x=inp["x"][perm], dy=inp["dy"][perm])
    out2 = O.layer_forward(inp2, 2)
    bwd2 = O.layer_backward(inp2, out2)
    np.testing.assert_allclose(out2["y"], out["y"][perm], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bwd2["dx"], bwd["dx"][perm], rtol=1e-12, atol=1e-14)
    assert (out2["counts"] == out["counts"]).all()
    for n in ("dw_gate", "dw_up", "dw_down", "dw_router"):
        np.testing.assert_allclose(bwd2[n], bwd[n], rtol=1e-10, atol=1e-14)


def test_random_routing_inputs_flow_through():
    wl, inp = tiny_inputs(T=64, d=8, E=8, k=4, f=6, routing="balanced")
    out = O.layer_forward(inp, 4)
    assert (out["counts"] == 64 * 4 // 8).all()
    np.testing.assert_array_equal(out["topk_idx"], inp["topk_idx"])
    assert "logits" not in out


def test_given_logits_override_routing():
    wl, inp = tiny_inputs(T=16, d=8, E=4, k=2)
    fake = np.tile(np.array([0.0, 1.0, 2.0, 3.0]), (16, 1))
    out = O.layer_forward(inp, 2, logits=fake)
    assert (out["topk_idx"] == np.array([3, 2])).all()
