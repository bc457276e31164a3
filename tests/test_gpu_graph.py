"""The layer's forward and backward captured once in a HIP graph (through
torch.cuda.graph) and replayed: every entry point only enqueues kernels on
the caller's stream (no allocation, no host synchronisation, no memset), so
each replay must reproduce the eagerly computed outputs bit for bit. Eager
work on other buffers runs between the replays."""
import numpy as np
import pytest
import torch

from moe_inputs import WORKLOADS, make_inputs

from gpu_util import dev

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_learned": ("bf16_e8", dict(T=600, d=256, f=192), "bf16"),
    "mxfp8_balanced": ("mxfp8_balanced", dict(T=512, d=256, E=16, f=256), "mxfp8"),
}

OUTS = ("y", "dx", "dw_gate", "dw_up", "dw_down", "dgate")


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_match_eager(case):
    from routing_grouped_gemm_softmax_amd import MoELayer
    name, over, dtype = CASES[case]
    wl = WORKLOADS[name].with_shape(**over)
    inp = make_inputs(wl, 0)
    print(f"[gpu] graph {case}: T={wl.T} d={wl.d} E={wl.E} k={wl.k} f={wl.f} {dtype}", flush=True)
    bf = torch.bfloat16
    t = {n: dev(inp[n], bf) for n in ("x", "dy", "w_gate", "w_up", "w_down")}
    learned = wl.routing == "learned"
    extra = {"w_router": dev(inp["w_router"], bf)} if learned else {
        "topk_idx": dev(inp["topk_idx"], torch.int32), "topk_gate": dev(inp["topk_gate"], torch.float32)}

    def step(layer):
        layer.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"], **extra)
        layer.backward(t["dy"])

    eager = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.f, dtype, learned_routing=learned)
    step(eager)
    torch.cuda.synchronize()
    ref = {n: getattr(eager, n).clone() for n in OUTS}
    if learned:
        ref["dw_router"] = eager.dw_router.clone()

    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.f, dtype, learned_routing=learned)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up launch outside the capture
        step(layer)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(layer)
    other = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.f, dtype, learned_routing=learned)
    for rep in range(3):
        for n in ref:
            getattr(layer, n).zero_()
        graph.replay()
        torch.cuda.synchronize()
        for n, r in ref.items():
            assert torch.equal(getattr(layer, n), r), (rep, n)
        step(other)  # eager work between replays
        torch.cuda.synchronize()
