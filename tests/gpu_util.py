"""Helpers for GPU parity tests: run the HIP layer on seeded inputs and
compare against the fp64 oracle with the per-tensor metric
err = max|gpu - ref| / max|ref|."""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as O

# Per-tensor tolerance on max|gpu - ref| / max|ref| for each storage dtype.
TOL = {"f32": 1e-5, "bf16": 2e-2, "mxfp8": 6e-2}


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def host(t) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().numpy()


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    den = np.abs(ref).max()
    num = np.abs(gpu - ref).max()
    if den == 0:
        return float(num)
    return float(num / den)


def torch_dtype(wl):
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


def run_layer(wl, inp, fwd_only=False, recompute=False):
    """Forward (+ backward) of the HIP layer on inputs from moe_inputs."""
    from routing_grouped_gemm_softmax_amd import MoELayer
    dt = torch_dtype(wl)
    learned = "w_router" in inp
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.f, wl.dtype, learned_routing=learned, recompute=recompute)
    t = {n: dev(inp[n], dt) for n in ("x", "dy", "w_gate", "w_up", "w_down")}
    if learned:
        t["w_router"] = dev(inp["w_router"], dt)
        layer.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"], w_router=t["w_router"])
    else:
        layer.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"],
                      topk_idx=dev(inp["topk_idx"], torch.int32), topk_gate=dev(inp["topk_gate"], torch.float32))
    if not fwd_only:
        layer.backward(t["dy"])
    torch.cuda.synchronize()
    return layer, t


def compare_layer(wl, inp, layer):
    k, tol = wl.k, TOL[wl.dtype]
    learned = "w_router" in inp
    gpu_logits = host(layer.logits).astype(np.float64) if learned else None
    ref = O.layer_forward(inp, k, logits=gpu_logits)
    refb = O.layer_backward(inp, ref)

    # Exact integer/byte results.
    np.testing.assert_array_equal(host(layer.topk_idx), ref["topk_idx"])
    np.testing.assert_array_equal(host(layer.counts), ref["counts"])
    np.testing.assert_array_equal(host(layer.offsets), ref["offsets"])
    np.testing.assert_array_equal(host(layer.row_of_slot), ref["row_of_slot"])
    np.testing.assert_array_equal(host(layer.token_of_row), ref["token_of_row"])
    np.testing.assert_array_equal(host(layer.xp), inp["x"][ref["token_of_row"]])

    G, U, H = (host(t) for t in layer.saved())
    pairs = {
        "gates": (host(layer.topk_gate), ref["gates"]),
        "G": (G, ref["G"]), "U": (U, ref["U"]), "H": (H, ref["H"]),
        "o": (host(layer.o), ref["O"]), "y": (host(layer.y), ref["y"]),
        "d_o": (host(layer.d_o), refb["dO"]), "dgate": (host(layer.dgate), refb["dgate"]),
        "dxp": (host(layer.dxp), refb["dXp"]),
        "dw_gate": (host(layer.dw_gate), refb["dw_gate"]), "dw_up": (host(layer.dw_up), refb["dw_up"]),
        "dw_down": (host(layer.dw_down), refb["dw_down"]), "dx": (host(layer.dx), refb["dx"]),
    }
    if learned:
        pairs["logits"] = (host(layer.logits), ref["logits"])
        pairs["dlogits"] = (host(layer.dlogits), refb["dlogits"])
        pairs["dw_router"] = (host(layer.dw_router), refb["dw_router"])
        # Top-k sets from the oracle's own fp64 logits may differ only at near-ties.
        own = O.topk_experts(ref["logits"], k)
        diff = (np.sort(own, 1) != np.sort(ref["topk_idx"], 1)).any(1)
        if diff.any():
            srt = np.sort(ref["logits"][diff], 1)[:, ::-1]
            assert (srt[:, k - 1] - srt[:, k] < 1e-5 * np.abs(ref["logits"]).max()).all()
    errs = {n: rel_err(g, r) for n, (g, r) in pairs.items()}
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"over tolerance {tol}: {bad}; all: {errs}"
    # Experts with no rows get exact zero weight gradients.
    for e in np.nonzero(ref["counts"] == 0)[0]:
        assert not host(layer.dw_gate)[e].any() and not host(layer.dw_down)[e].any()
    return errs
