"""bench.py's command-line contract on a host without a GPU: more than one
GPU is refused with a message (the library has no multi-GPU path), and the
algorithmic work it reports per call follows the layer's formulas."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_work_formulas():
    import bench
    from moe_inputs import WORKLOADS
    wl = WORKLOADS["bf16_e8"]
    T, d, E, k, f = wl.T, wl.d, wl.E, wl.k, wl.f
    S = T * k
    w = bench.algorithmic_work(wl)
    assert w["moe_grouped_ffn_fwd"]["flops"] + w["moe_grouped_ffn_bwd"]["flops"] == 18 * S * d * f
    assert w["moe_dispatch"]["bytes"] == (1 + k) * T * d * 2
    assert w["moe_combine_bwd"]["bytes"] == (1 + 2 * k) * T * d * 2
    assert w["moe_route"]["flops"] == 2 * T * d * E
    mx = bench.algorithmic_work(WORKLOADS["mxfp8_balanced"])
    wm = WORKLOADS["mxfp8_balanced"]
    Sm = wm.T * wm.k
    # the MXFP8 images of xp and d_o: one byte per element plus one per 32
    # x read once; xp written only as its two MXFP8 operands
    assert mx["moe_dispatch"]["bytes"] == wm.T * wm.d * 2 + 2 * (Sm * wm.d + Sm * wm.d // 32)
    assert "moe_route" not in mx
    rc = bench.algorithmic_work(wl, recompute=True)
    assert rc["moe_grouped_ffn_bwd"]["flops_recompute"] == 4 * S * d * f


def test_gemm_combined_roofline_floors():
    """The 128-expert layer's grouped GEMMs are HBM-bound (floor 0.814 ms: the
    weights read twice and their gradients written, plus activations) while
    the 8-expert layer's are MFMA-bound (0.495 ms)."""
    import bench
    from moe_inputs import WORKLOADS
    e8, e128 = WORKLOADS["bf16_e8"], WORKLOADS["bf16_e128"]
    fl = 18 * e8.T * e8.k * e8.d * e8.f
    assert abs(fl / 2.5e15 * 1e3 - 0.4948) < 1e-3
    assert bench.gemm_compulsory_bytes(e8) / 8e12 < fl / 2.5e15
    assert abs(bench.gemm_compulsory_bytes(e128) / 8e12 * 1e3 - 0.8137) < 1e-3


def test_gemm_step_flops_sum_to_the_layer():
    """The five grouped-GEMM steps the kernel timer surveys add up to the
    layer's 18*S*d*f (22*S*d*f with the recomputed gate/up GEMM)."""
    import bench
    from moe_inputs import WORKLOADS
    wl = WORKLOADS["mxfp8_balanced"]
    u = wl.T * wl.k * wl.d * wl.f
    assert sum(bench.gemm_mode_flops(wl).values()) == 18 * u
    assert sum(bench.gemm_mode_flops(wl, recompute=True).values()) == 22 * u
    assert bench.GEMM_MODE_NAMES == tuple(__import__("routing_grouped_gemm_softmax_amd").GEMM_MODES)


def test_cpu_baseline_mxfp8_sample_runs():
    """The per-expert MXFP8 sample of the CPU baseline, on a small shape."""
    import bench
    from moe_inputs import WORKLOADS, make_inputs
    wl = WORKLOADS["mxfp8_balanced"].with_shape(T=256, d=128, E=16, f=128)
    r = bench.cpu_baseline(wl, make_inputs(wl, 0), budget_s=1.0)
    assert r["value"] > 0 and r["kind"] == "oracle" and r["cores"] >= 1 and r["cpu_model"]
    assert "whole experts" in r["sample"]


def test_source_hash_ignores_comments_only():
    """The kernel-source fingerprint that dates the traffic counters changes
    with the code, not with its comments."""
    import bench
    a = b'#include "x.h"\n// one\nint f(int v) { return v + 1; }  /* two */\n'
    b = b'#include "x.h"\n/* other\n text */\nint f(int v) { return v + 1; }\n\n// more\n'
    c = b'#include "x.h"\nint f(int v) { return v + 2; }\n'
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    assert b'"x.h"' in bench._code_only(a)
