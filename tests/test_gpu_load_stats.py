"""GPU expert-load diagnostics (moe_load_stats) against the oracle's
load_stats on counts from the device's own dispatch: integer figures exact,
fp64 figures within 1e-12 relative (summation order and the log routine
differ), reruns bit-identical."""
import numpy as np
import pytest
import torch

from moe_inputs import WORKLOADS, make_inputs
from oracle import moe_oracle as O

from gpu_util import dev, host, run_layer

pytestmark = pytest.mark.gpu

CASES = {
    "zipf_empty_experts": ("bf16_zipf", dict(T=256, d=128, E=16, f=128), [1, 0, 2, 1, 1, 0, 3, 1, 1, 1, 0, 1, 2, 1, 1, 0]),
    "balanced_E128": ("mxfp8_balanced", dict(T=1024, d=128, E=128, f=128, dtype="bf16"), None),
    "learned_E8": ("bf16_e8", dict(T=600, d=256, f=128), None),
    "dense_E1": ("tiny_f32", dict(T=100, E=1, k=1), None),
    "zipf_E256": ("bf16_zipf", dict(T=512, d=128, E=256, f=128), None),
}


def _check(stats, counts):
    g = host(stats)
    r = O.load_stats(counts)
    print("gpu:", dict(zip(O.LOAD_STATS, np.round(g, 6))), flush=True)
    np.testing.assert_array_equal(g[[0, 1, 6]], r[[0, 1, 6]])
    np.testing.assert_allclose(g, r, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("case", list(CASES))
def test_load_stats_match_oracle(case):
    name, over, pop = CASES[case]
    wl = WORKLOADS[name].with_shape(**over)
    inp = make_inputs(wl, 5, popularity=pop)
    print(f"[gpu] load stats {case}: T={wl.T} E={wl.E} k={wl.k}", flush=True)
    layer, _ = run_layer(wl, inp, fwd_only=True)
    stats = layer.load_stats()
    torch.cuda.synchronize()
    a = host(stats).copy()
    _check(stats, host(layer.counts))
    layer.load_stats()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(layer.stats), a)


def test_load_stats_of_no_rows_and_one_hot():
    import routing_grouped_gemm_softmax_amd as M
    out = torch.empty(8, dtype=torch.float64, device="cuda")
    for c in (np.zeros(16, np.int32), np.eye(1, 64, 17, dtype=np.int32)[0] * 4096):
        print(f"[gpu] load stats counts sum={c.sum()} E={c.size}", flush=True)
        M.moe_load_stats(dev(c, torch.int32), out)
        torch.cuda.synchronize()
        _check(out, c)
