"""Router top-k on exact ties (GPU), through the C ABI's moe_route.

Each token activates the k experts with the largest logits; the selection
rule breaks equal logits toward the lower expert index (the oracle's
topk_experts, pinned on the CPU against brute force with ties). Router weights
whose columns repeat give exactly equal logits, so these cases exercise the
tie-break in every top-k layout the bf16 router uses (expert blocks of 16, 1
to 16 per lane), including the all-equal case where the first k experts win.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import routing_grouped_gemm_softmax_amd._lib as L
from oracle import moe_oracle as O

from gpu_util import dev, host

pytestmark = pytest.mark.gpu


def _route(x, w, T, d, E, k, dtype):
    shape = L.MoeShape.make(T, d, E, k, 64, dtype)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    xs, ws_ = dev(x, tdt), dev(w, tdt)
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gate = torch.empty(T, k, dtype=torch.float32, device="cuda")
    n = L.workspace_size(L.MOE_OP_ROUTE, shape)
    wsp = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    L.moe_route(xs, ws_, shape, logits, idx, gate, wsp)
    torch.cuda.synchronize()
    return host(logits), host(idx), host(gate)


@pytest.mark.parametrize("dtype,E,k,d,rep", [
    ("bf16", 8, 4, 512, 2),     # pairs of equal experts, one 16-expert block
    ("bf16", 16, 8, 256, 4),    # groups of four
    ("bf16", 32, 3, 128, 2),    # two blocks
    ("bf16", 128, 4, 2048, 2),  # eight blocks
    ("bf16", 256, 8, 128, 8),   # sixteen blocks, groups of eight
    ("bf16", 128, 8, 256, 128), # every logit of a token equal
    ("f32", 64, 4, 128, 2),     # the fp32 router's one-token-per-wave selection
])
def test_route_ties_go_to_the_lower_index(dtype, E, k, d, rep):
    print(f"route ties: {dtype} E={E} k={k} d={d} groups of {rep}", flush=True)
    rng = np.random.default_rng(1000 * E + 10 * k + rep)
    T = 77
    x = rng.standard_normal((T, d))
    w = np.repeat(rng.standard_normal((d, E // rep)) * 0.05, rep, axis=1)
    logits, idx, gate = _route(x, w, T, d, E, k, dtype)
    # Equal columns give bitwise equal logits, so the cases really tie.
    for j in range(1, rep):
        np.testing.assert_array_equal(logits[:, j::rep], logits[:, 0::rep])
    ref_idx, ref_gate = O.route(logits.astype(np.float64), k)
    np.testing.assert_array_equal(idx, ref_idx)
    np.testing.assert_allclose(gate, ref_gate, rtol=0, atol=1e-6)
    if rep == E:
        np.testing.assert_array_equal(idx, np.tile(np.arange(k, dtype=np.int32), (T, 1)))
