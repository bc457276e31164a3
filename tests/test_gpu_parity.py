"""GPU parity of the whole layer (forward + backward) against the fp64 oracle.

Bit-exact: top-k indices, counts, offsets, row_of_slot, token_of_row and the
bytes of xp. Tolerance (max|gpu-ref| / max|ref| per tensor): 1e-5 for fp32
layers, 2e-2 for bf16 layers. Routing is compared on identical logits: the
oracle routes from the GPU's fp32 logits widened to fp64, while the logits
themselves are compared with the oracle's own fp64 x W_r.
"""
import numpy as np
import pytest
import torch

from moe_inputs import WORKLOADS, make_inputs
from oracle import moe_oracle as O

from gpu_util import TOL, compare_layer, dev, host, rel_err, run_layer

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, shape overrides, zipf popularity override)
    "tiny_f32_full": ("tiny_f32", {}, None),
    "f32_dense_E1_k1": ("tiny_f32", dict(T=100, E=1, k=1), None),
    "f32_k_equals_E": ("tiny_f32", dict(T=77, E=6, k=6, f=64), None),
    "f32_ragged_many_tiles": ("tiny_f32", dict(T=333, d=128, E=4, k=2, f=192), None),
    "bf16_e8_ragged": ("bf16_e8", dict(T=600, d=256, f=192), None),
    "bf16_e128_small_experts": ("bf16_e128", dict(T=300, d=128, f=128), None),
    "bf16_k1": ("bf16_e8", dict(T=200, d=128, f=64, k=1), None),
    "bf16_zipf_random": ("bf16_zipf", dict(T=512, d=256, E=32, f=128), None),
    "bf16_zipf_empty_experts": ("bf16_zipf", dict(T=256, d=128, E=16, f=128),
                                [1, 0, 2, 1, 1, 0, 3, 1, 1, 1, 0, 1, 2, 1, 1, 0]),
    "bf16_balanced": ("mxfp8_balanced", dict(T=256, d=128, E=16, f=128, dtype="bf16"), None),
    # 256 x 256 tiles on the persistent streaming kernels: several tiles per
    # workgroup (512 tiles in FWD_GU and FWD_DOWN), ragged expert ends, and a
    # short last round left to quarter tiles.
    "bf16_stream_multi_tile": ("bf16_e8", dict(T=16384, d=1024, E=4, k=2, f=512), None),
    # 256 x 256 tiles with an empty expert.
    "bf16_stream_empty_expert": ("bf16_zipf", dict(T=4096, d=512, E=4, k=2, f=512), [1, 0, 2, 1]),
    # Streaming weight gradients (experts average 64 rows): tiles of 0 to a few
    # slabs, several epilogues within three slabs, two tiles per workgroup.
    # Eight experts get no rows.
    "bf16_wgrad_stream_short_tiles": ("bf16_zipf", dict(T=4096, d=512, E=128, k=2, f=256),
                                      [0 if e % 16 == 5 else 1 + e % 7 for e in range(128)]),
    # 512 rows per expert on average with skewed loads: every expert's whole
    # 256-row bands in 256 x 256 tiles, the rest in 128 x 256 tiles (two
    # launches per row-ragged step): loads from 1991 rows (seven bands) down
    # to 252 (a remainder only), and an empty expert.
    "bf16_zipf_row_bands": ("bf16_zipf", dict(T=2048, d=256, E=16, f=256),
                            [30, 9, 4, 2, 1, 1, 1, 1, 0, 1, 1, 1, 1, 1, 1, 1]),
    # The largest expert count and top-k the library takes, learned routing:
    # about 9 rows per expert, 16 router column blocks, eight slots per token.
    # d and f odd multiples of 128 at about 1024 rows per expert: 256 x 128
    # tiles (and their quarter-tile tails) for the down forward, down dgrad
    # and gate/up dgrad; 128-row weight-gradient tiles.
    "bf16_256x128_tiles": ("bf16_e8", dict(T=2048, d=384, f=640), None),
    # 128-row tiles (about 256 rows per expert) around one expert of 1541
    # rows: its 13 row tiles form tile groups of 8 and 5, the other experts'
    # groups hold 2 to 5; the last expert gets no rows.
    "bf16_128row_tiles_hot_expert": ("bf16_zipf", dict(T=2048, d=256, E=32, f=256), [6, 1.5] + [0.5] * 29 + [0]),
    "bf16_max_E256_k8": ("bf16_e8", dict(T=300, d=128, E=256, k=8, f=128), None),
    # The router at wider d: a ragged last block of 16 tokens at d = 512, and
    # d = 4096 with eight 16-expert blocks (32 k steps per wave).
    "bf16_router_ragged_d512": ("bf16_e8", dict(T=300, d=512, E=8, k=2, f=128), None),
    "bf16_router_d4096_E128": ("bf16_e128", dict(T=77, d=4096, E=128, f=64), None),
    # One token.
    "bf16_single_token": ("bf16_e8", dict(T=1, d=128, E=8, k=4, f=64), None),
    "f32_single_token_k8": ("tiny_f32", dict(T=1, E=8, k=8), None),
}


@pytest.mark.parametrize("case", list(CASES))
def test_layer_matches_oracle(case):
    name, over, pop = CASES[case]
    wl = WORKLOADS[name].with_shape(**over)
    inp = make_inputs(wl, 0, popularity=pop)
    print(f"[gpu] {case}: T={wl.T} d={wl.d} E={wl.E} k={wl.k} f={wl.f} {wl.dtype} {wl.routing}", flush=True)
    layer, _ = run_layer(wl, inp)
    errs = compare_layer(wl, inp, layer)
    print({n: f"{e:.2e}" for n, e in errs.items()}, flush=True)


def test_rerun_is_bit_identical():
    wl = WORKLOADS["bf16_e8"].with_shape(T=600, d=256, f=192)
    inp = make_inputs(wl, 1)
    a, _ = run_layer(wl, inp)
    outs_a = [host(t).copy() for t in (a.y, a.dx, a.dw_gate, a.dw_down, a.dw_router, a.dlogits)]
    b, _ = run_layer(wl, inp)
    outs_b = [host(t) for t in (b.y, b.dx, b.dw_gate, b.dw_down, b.dw_router, b.dlogits)]
    for x, y in zip(outs_a, outs_b):
        np.testing.assert_array_equal(x, y)


def test_identity_experts_through_dispatch_and_combine():
    # Combine applied to xp itself (identity experts): y = sum_j g_tj x_t = x_t.
    import routing_grouped_gemm_softmax_amd as M
    wl = WORKLOADS["tiny_f32"].with_shape(T=300, d=128, E=8, k=3)
    inp = make_inputs(wl, 2)
    layer, t = run_layer(wl, inp, fwd_only=True)
    y = torch.empty_like(t["x"])
    M.moe_combine(layer.xp, layer.topk_gate, layer.row_of_slot, layer.shape, y)
    torch.cuda.synchronize()
    assert rel_err(host(y), inp["x"]) < 1e-6


def test_invalid_expert_id_sets_status_and_is_not_routed():
    import routing_grouped_gemm_softmax_amd as M
    wl = WORKLOADS["bf16_zipf"].with_shape(T=128, d=64, E=8, f=64)
    inp = make_inputs(wl, 3, weights=False)
    idx = inp["topk_idx"].copy()
    idx[5, 2] = 8      # out of range
    idx[70, 0] = -1    # negative
    layer = M.MoELayer(wl.T, wl.d, wl.E, wl.k, wl.f, "bf16", learned_routing=False)
    x = dev(inp["x"], torch.bfloat16)
    M.moe_dispatch(x, dev(idx, torch.int32), layer.shape, layer.counts, layer.offsets, layer.row_of_slot,
                   layer.token_of_row, layer.xp, layer.ws_dispatch)
    status = M.moe_read_device_status(layer.ws_dispatch)
    assert status == 1
    rs = host(layer.row_of_slot)
    assert rs[5, 2] == -1 and rs[70, 0] == -1
    assert host(layer.offsets)[-1] == wl.T * wl.k - 2
    # A clean dispatch resets the status word.
    M.moe_dispatch(x, dev(inp["topk_idx"], torch.int32), layer.shape, layer.counts, layer.offsets,
                   layer.row_of_slot, layer.token_of_row, layer.xp, layer.ws_dispatch)
    assert M.moe_read_device_status(layer.ws_dispatch) == 0


@pytest.mark.parametrize("case", ["f32_ragged_many_tiles", "bf16_e8_ragged", "bf16_zipf_empty_experts",
                                  "bf16_stream_multi_tile"])
def test_recompute_matches_oracle_and_saved_layer(case):
    """Activation recompute (MOE_FLAG_RECOMPUTE): the layer saves no G, U, H,
    the backward rebuilds them, and every output matches the oracle and is
    bit-identical to the layer that saves them."""
    name, over, pop = CASES[case]
    wl = WORKLOADS[name].with_shape(**over)
    inp = make_inputs(wl, 4, popularity=pop)
    print(f"[gpu] recompute {case}: T={wl.T} d={wl.d} E={wl.E} k={wl.k} f={wl.f} {wl.dtype}", flush=True)
    rec, _ = run_layer(wl, inp, recompute=True)
    assert rec.save.numel() == 0
    errs = compare_layer(wl, inp, rec)
    print({n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
    ref, _ = run_layer(wl, inp)
    for n in ("o", "y", "d_o", "dgate", "dxp", "dw_gate", "dw_up", "dw_down", "dx"):
        assert torch.equal(getattr(rec, n), getattr(ref, n)), n
    for a, b in zip(rec.saved(), ref.saved()):
        assert torch.equal(a, b)


def test_duplicate_expert_in_a_token_sets_status():
    """A token that names one expert in two slots sets MOE_DEV_DUP_EXPERT; both
    slots are still routed, to consecutive rows of that expert, as the
    oracle's stable counting sort places them. An out-of-range id beside it
    sets MOE_DEV_BAD_EXPERT too."""
    import routing_grouped_gemm_softmax_amd as M
    wl = WORKLOADS["bf16_zipf"].with_shape(T=700, d=64, E=8, f=64)
    inp = make_inputs(wl, 5, weights=False)
    idx = inp["topk_idx"].copy()
    idx[9] = [3, 3, 1, 2]
    idx[650] = [0, 5, 7, 5]
    layer = M.MoELayer(wl.T, wl.d, wl.E, wl.k, wl.f, "bf16", learned_routing=False)
    x = dev(inp["x"], torch.bfloat16)

    def run(ids):
        M.moe_dispatch(x, dev(ids, torch.int32), layer.shape, layer.counts, layer.offsets, layer.row_of_slot,
                       layer.token_of_row, layer.xp, layer.ws_dispatch)
        return M.moe_read_device_status(layer.ws_dispatch)

    assert run(idx) == M._lib.MOE_DEV_DUP_EXPERT
    counts, offsets, rs, tor = O.dispatch_plan(idx, wl.E)
    np.testing.assert_array_equal(host(layer.counts), counts)
    np.testing.assert_array_equal(host(layer.row_of_slot), rs)
    np.testing.assert_array_equal(host(layer.token_of_row), tor)
    assert host(layer.row_of_slot)[9, 1] == host(layer.row_of_slot)[9, 0] + 1
    idx2 = idx.copy()
    idx2[100, 3] = 8
    assert run(idx2) == M._lib.MOE_DEV_DUP_EXPERT | M._lib.MOE_DEV_BAD_EXPERT
    assert run(inp["topk_idx"]) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,E", [(64, 8), (512, 128)], ids=["narrow_rows", "wave_rows_E128"])
def test_dispatch_bwd_dense_dlogits(dtype, d, E):
    """moe_dispatch_bwd with dlogits rows that have more than k non-zeros (a
    caller's dense router gradient): dx = sum_j dxp[row(t,j)] + dlogits[t] W_r^T
    over every column. Rows with k or fewer non-zeros take the fast path;
    rows with exactly k + 1 and with all E non-zero take the dense one."""
    import routing_grouped_gemm_softmax_amd as M
    k = 4
    wl = WORKLOADS["bf16_e8"].with_shape(T=300, d=d, E=E, k=k, f=64, dtype=dtype)
    inp = make_inputs(wl, 6, weights=False)
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((wl.T, E))
    idx = O.topk_experts(logits, k)
    counts, offsets, rs, tor = O.dispatch_plan(idx, E)
    S = wl.T * k
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    dxp = rng.standard_normal((S, d)).astype(np.float32)
    if dtype == "bf16":
        from moe_inputs import bf16_round
        dxp = bf16_round(dxp)
    dl = np.zeros((wl.T, E), dtype=np.float32)
    np.put_along_axis(dl, idx.astype(np.int64), rng.standard_normal((wl.T, k)).astype(np.float32), axis=1)
    dl[0::3] = rng.standard_normal((len(dl[0::3]), E)).astype(np.float32)           # all E non-zero
    extra = [t for t in range(1, wl.T, 3)]
    for t in extra:                                                                   # exactly k + 1
        off = [e for e in range(E) if e not in idx[t]][0]
        dl[t, off] = 0.5
    shape = M.MoeShape.make(wl.T, d, E, k, 64, dtype)
    ws = torch.empty(max(M.workspace_size(M._lib.MOE_OP_DISPATCH_BWD, shape), 256), dtype=torch.uint8,
                     device="cuda")
    dx = torch.empty(wl.T, d, dtype=tdt, device="cuda")
    print(f"[gpu] dense dlogits {dtype} d={d} E={E}", flush=True)
    M.moe_dispatch_bwd(dev(dxp, tdt), dev(rs, torch.int32), dev(dl, torch.float32), dev(inp["w_router"], tdt),
                       shape, dx, ws)
    torch.cuda.synchronize()
    want = O.dispatch_backward(dxp, rs, dl.astype(np.float64) @ np.asarray(inp["w_router"], np.float64).T)
    err = rel_err(host(dx), want)
    print(f"dx err {err:.2e}", flush=True)
    assert err <= TOL[dtype], err
