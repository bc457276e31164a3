"""Pins for the oracle's backward pass.

Two independent references: (1) torch autograd in fp64 on a dense
formulation of the layer (every expert applied to every token, combined
through a gate matrix that is zero off the routed set); (2) central finite
differences of the oracle's own forward. Plus closed-form invariants.
"""
import numpy as np
import pytest
import torch

from moe_inputs import WORKLOADS, make_inputs
from oracle import moe_oracle as O


def tiny(T=24, d=8, E=4, k=2, f=6, seed=0, routing="learned"):
    wl = WORKLOADS["tiny_f32"].with_shape(T=T, d=d, E=E, k=k, f=f, routing=routing)
    return make_inputs(wl, seed)


def dense_autograd(inp, k):
    """fp64 torch: y = sum_e Gmask[t,e] * FFN_e(x_t); routing mask held fixed."""
    t = {n: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True)
         for n, v in inp.items() if n in ("x", "w_router", "w_gate", "w_up", "w_down")}
    logits = t["x"] @ t["w_router"]
    idx = O.topk_experts(logits.detach().numpy(), k)
    mask = torch.zeros_like(logits, dtype=torch.bool)
    mask[torch.arange(logits.shape[0])[:, None], torch.tensor(idx, dtype=torch.long)] = True
    gate = torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=1)
    y = torch.zeros_like(t["x"])
    for e in range(t["w_gate"].shape[0]):
        h = torch.nn.functional.silu(t["x"] @ t["w_gate"][e]) * (t["x"] @ t["w_up"][e])
        y = y + gate[:, e:e + 1] * (h @ t["w_down"][e])
    loss = (y * torch.tensor(np.asarray(inp["dy"], dtype=np.float64))).sum()
    loss.backward()
    return y.detach().numpy(), {n: v.grad.numpy() for n, v in t.items()}


@pytest.mark.parametrize("T,E,k,seed", [(24, 4, 2, 0), (40, 8, 4, 1), (16, 3, 3, 2), (30, 6, 1, 3)])
def test_backward_matches_autograd(T, E, k, seed):
    inp = tiny(T=T, E=E, k=k, seed=seed)
    fwd = O.layer_forward(inp, k)
    bwd = O.layer_backward(inp, fwd)
    y_ref, g = dense_autograd(inp, k)
    np.testing.assert_allclose(fwd["y"], y_ref, rtol=1e-11, atol=1e-14)
    for ours, ref in (("dx", "x"), ("dw_router", "w_router"), ("dw_gate", "w_gate"),
                      ("dw_up", "w_up"), ("dw_down", "w_down")):
        scale = np.abs(g[ref]).max() + 1e-300
        assert np.abs(bwd[ours] - g[ref]).max() / scale < 1e-11, ours


def _loss(inp, k):
    return float((O.layer_forward(inp, k)["y"] * inp["dy"]).sum())


def test_finite_differences():
    k = 2
    inp = {n: (v.astype(np.float64) if v.dtype.kind == "f" else v) for n, v in tiny(T=12, E=4, k=k, seed=5).items()}
    fwd = O.layer_forward(inp, k)
    bwd = O.layer_backward(inp, fwd)
    l = fwd["logits"]
    srt = np.sort(l, axis=1)[:, ::-1]
    assert (srt[:, k - 1] - srt[:, k]).min() > 1e-4  # routing stays fixed under +-h
    h = 1e-6
    rng = np.random.default_rng(0)
    for name, grad in (("x", "dx"), ("w_router", "dw_router"), ("w_gate", "dw_gate"),
                       ("w_up", "dw_up"), ("w_down", "dw_down")):
        a = inp[name]
        for flat in rng.choice(a.size, size=6, replace=False):
            pos = np.unravel_index(flat, a.shape)
            old = a[pos]
            a[pos] = old + h; lp = _loss(inp, k)
            a[pos] = old - h; lm = _loss(inp, k)
            a[pos] = old
            fd = (lp - lm) / (2 * h)
            an = bwd[grad][pos]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, pos, fd, an)


def test_router_gradient_invariants():
    inp = tiny(T=50, E=8, k=3, seed=7)
    fwd = O.layer_forward(inp, 3)
    bwd = O.layer_backward(inp, fwd)
    dl = bwd["dlogits"]
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-14)
    off = np.ones_like(dl, dtype=bool)
    np.put_along_axis(off, fwd["topk_idx"].astype(np.int64), False, axis=1)
    assert (dl[off] == 0).all()


def test_k1_has_no_router_gradient():
    inp = tiny(T=20, E=4, k=1, seed=8)
    fwd = O.layer_forward(inp, 1)
    bwd = O.layer_backward(inp, fwd)
    assert (bwd["dlogits"] == 0).all() and (bwd["dw_router"] == 0).all()


def test_k_equals_E_router_gradient_is_softmax_jacobian():
    inp = tiny(T=10, E=4, k=4, seed=9)
    fwd = O.layer_forward(inp, 4)
    bwd = O.layer_backward(inp, fwd)
    lt = torch.tensor(fwd["logits"], requires_grad=True)
    p = torch.softmax(lt, dim=1)
    # dgate is aligned with topk_idx; scatter it back to expert order.
    dg = np.zeros_like(fwd["logits"])
    np.put_along_axis(dg, fwd["topk_idx"].astype(np.int64), bwd["dgate"], axis=1)
    (p * torch.tensor(dg)).sum().backward()
    np.testing.assert_allclose(bwd["dlogits"], lt.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_empty_expert_has_zero_weight_gradient():
    wl = WORKLOADS["tiny_f32"].with_shape(T=32, d=8, E=6, k=2, f=6, routing="zipf")
    pop = np.array([1.0, 0.0, 2.0, 1.0, 0.0, 1.0])
    inp = make_inputs(wl, 0, popularity=pop)
    fwd = O.layer_forward(inp, 2)
    bwd = O.layer_backward(inp, fwd)
    assert fwd["counts"][1] == 0 and fwd["counts"][4] == 0
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert (bwd[n][1] == 0).all() and (bwd[n][4] == 0).all()
        assert np.abs(bwd[n][0]).max() > 0


def test_linear_in_upstream_gradient():
    inp = tiny(T=20, E=4, k=2, seed=10)
    fwd = O.layer_forward(inp, 2)
    b1 = O.layer_backward(inp, fwd)
    b2 = O.layer_backward(inp, fwd, dy=-3.0 * inp["dy"].astype(np.float64))
    for n in ("dx", "dw_gate", "dw_up", "dw_down", "dw_router", "dgate"):
        np.testing.assert_allclose(b2[n], -3.0 * b1[n], rtol=1e-12, atol=1e-15)
