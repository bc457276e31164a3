"""Whole-layer GPU parity at the full workload sizes, in the launch
configuration the benchmark times (MoELayer with its preallocated buffers).
Every element of every output is compared with the fp64 oracle."""
import pytest

from moe_inputs import WORKLOADS, make_inputs

from gpu_util import compare_layer, run_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["bf16_e8", "bf16_e128"])
def test_full_size_layer(name):
    wl = WORKLOADS[name]
    print(f"[gpu] full size {name}: T={wl.T} d={wl.d} E={wl.E} k={wl.k} f={wl.f}", flush=True)
    inp = make_inputs(wl, 0)
    layer, _ = run_layer(wl, inp)
    errs = compare_layer(wl, inp, layer)
    print({n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
