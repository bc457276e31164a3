"""Benchmark: MoE expert layer forward + backward on one MI355X.

One step = the whole hot path on one batch: route, dispatch, grouped SwiGLU
FFN forward, combine, then combine backward, grouped FFN backward (dgrad and
wgrad), router backward and dispatch backward. Inputs are seeded synthetic
tensors already resident in HBM. The default workload is the largest
single-GPU configuration: the MXFP8 layer with 128 experts and balanced
random routing (T=32768, d_model=4096, top-4, d_ff=1536), with the bf16 path
of the same shape timed beside it for the MXFP8/bf16 ratio.

Prints one JSON line: tokens/s for the step, the grouped-GEMM TFLOP/s,
dispatch/combine GB/s, a roofline object for the dominant grouped-GEMM
kernel (its launches timed with HIP events that the library records on the
stream it launches on) and the fp64 oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (MXFP8 grouped GEMMs)
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (MFMA / packed vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


_C_COMMENT = re.compile(rb'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"', re.S)


def _code_only(text: bytes) -> bytes:
    """C/C++ source without its comments and blank space at line ends or
    between lines (string literals kept), so that a change to a comment
    leaves the hash alone."""
    text = _C_COMMENT.sub(lambda m: m.group(0) if m.group(0).startswith(b'"') else b" ", text)
    lines = (ln.rstrip() for ln in text.splitlines())
    return b"\n".join(ln for ln in lines if ln)


def kernel_source_hash(files=None) -> str:
    """Hash of the library's kernel sources, comments left out (all of csrc,
    or the listed files plus the build script, whose flags shape the code)."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "routing_grouped_gemm_softmax_amd")
    csrc = os.path.join(pkg, "csrc")
    names = sorted(os.listdir(csrc)) if files is None else sorted(files)
    for n in names:
        with open(os.path.join(csrc, n), "rb") as fh:
            h.update(n.encode() + _code_only(fh.read()))
    if files is not None:
        with open(os.path.join(pkg, "build.py"), "rb") as fh:
            h.update(b"build.py" + fh.read())
    return h.hexdigest()[:16]


# Sources each grouped-GEMM kernel family is compiled from.
GEMM_SOURCES = {
    "mxfp8": ["gemm_mx.hip", "gemm_device.h", "grouped_gemm.h", "common.h", "mx_encode.h", "kernels.h"],
    "bf16": ["gemm_bf16.hip", "gemm_device.h", "grouped_gemm.h", "common.h", "mx_encode.h", "kernels.h"],
    "f32": ["gemm.hip", "grouped_gemm.h", "common.h", "kernels.h"],
}
GEMM_MODE_NAMES = ("fwd_gu", "fwd_down", "bwd_down", "bwd_gu", "wgrad")


def gemm_mode_flops(wl, recompute=False):
    """Algorithmic flops per step of each grouped-GEMM step (both weight
    gradients together for wgrad; the recomputed gate/up GEMM adds to fwd_gu)."""
    S, d, f = wl.T * wl.k, wl.d, wl.f
    u = S * d * f
    return {"fwd_gu": (8 if recompute else 4) * u, "fwd_down": 2 * u, "bwd_down": 2 * u, "bwd_gu": 4 * u,
            "wgrad": 6 * u}


def algorithmic_work(wl, recompute=False):
    """FLOPs and HBM bytes the method must move, per library call, per step.
    With activation recompute the backward also runs the gate/up GEMM again
    (flops_recompute); TFLOP/s figures count only the method's 18*S*d*f."""
    T, d, E, k, f = wl.T, wl.d, wl.E, wl.k, wl.f
    S = T * k
    b = 4 if wl.dtype == "f32" else 2
    work = {
        "moe_grouped_ffn_fwd": {"flops": 6 * S * d * f},
        "moe_grouped_ffn_bwd": {"flops": 12 * S * d * f},
        # token-major copies: read the token row once, write/read k routed rows
        "moe_dispatch": {"bytes": (1 + k) * T * d * b},
        "moe_combine": {"bytes": (1 + k) * T * d * b},
        "moe_combine_bwd": {"bytes": (1 + 2 * k) * T * d * b},
        "moe_dispatch_bwd": {"bytes": (1 + k) * T * d * b},
    }
    if wl.dtype == "mxfp8":
        # dispatch writes xp only as its two MXFP8 operands (along d, and
        # along each expert's tokens; one E4M3 byte per element plus one E8M0
        # byte per 32), not as rows: it reads x and writes the two images.
        # Likewise combine backward writes dO only as its two operands: it
        # reads dy and o and writes the two images.
        work["moe_dispatch"]["bytes"] = T * d * b + 2 * (S * d + S * d // 32)
        work["moe_combine_bwd"]["bytes"] = (1 + k) * T * d * b + 2 * (S * d + S * d // 32)
    if recompute:
        work["moe_grouped_ffn_bwd"]["flops_recompute"] = 4 * S * d * f
    if wl.routing == "learned":
        work["moe_route"] = {"flops": 2 * T * d * E}
        work["moe_route_bwd"] = {"flops": 2 * T * d * E}
    return work


def gemm_compulsory_bytes(wl):
    """HBM bytes the two grouped-FFN calls cannot avoid in one forward+backward
    (bf16 and fp32 layers; every tensor read or written once per use):
    forward   read Xp, W_gate, W_up, W_down, H (down GEMM); write G, U, H, O;
    backward  read dO, G, U, the three weights, dG|dU (gate/up dgrad), H and
              dO (dW_down), Xp and dG|dU (dW_gate|dW_up); write dG|dU, dXp and
              the three weight gradients."""
    T, d, E, k, f = wl.T, wl.d, wl.E, wl.k, wl.f
    S, b = T * k, (4 if wl.dtype == "f32" else 2)
    W = 3 * E * d * f
    fwd = S * d + W + S * f + 3 * S * f + S * d
    bwd = (S * d + 2 * S * f + W + 2 * S * f + S * f + S * d + S * d + 2 * S * f
           + 2 * S * f + S * d + W)
    return (fwd + bwd) * b


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inp, budget_s: float = 20.0):
    """The fp64 oracle (as it stands) on a bounded sample of the same
    workload, on the host cores; the rate is scaled to whole-layer tokens/s.

    bf16 and fp32 layers: when a full forward+backward would take far longer
    than ``budget_s`` of CPU time, the oracle runs on the first T' tokens of
    the same inputs (same d, E, k, f and weights; T' from an fp64 rate
    estimate). MXFP8 layers quantise every expert's weights in every call
    whatever T', so the sample is per expert instead: the oracle's MXFP8 FFN
    forward and backward of a few whole experts' rows with their weights,
    plus the layer's token-level steps (dispatch plan, gather, combine and
    their backward) on the same share of the tokens, scaled by E / experts."""
    from threadpoolctl import threadpool_info

    from moe_inputs import make_inputs
    from oracle import moe_oracle as O
    import numpy as np
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    host = {"cores": threads, "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
    if wl.dtype == "mxfp8":
        E, k, T = wl.E, wl.k, wl.T
        idx, gates = inp["topk_idx"], inp["topk_gate"].astype(np.float64)
        t0 = time.perf_counter()
        counts, offsets, row_of_slot, token_of_row = O.dispatch_plan(idx, E)
        t_plan = time.perf_counter() - t0
        n_e, t_ffn, e = 0, 0.0, 0
        while e < E and (n_e < 2 or t_ffn < budget_s * 0.5) and n_e < 8:
            a, b = int(offsets[e]), int(offsets[e + 1])
            if a < b:
                rows = np.arange(a, b)
                tok = token_of_row[rows]
                slot = np.argmax(row_of_slot[tok] == rows[:, None], axis=1)
                one = np.array([0, b - a])
                w = tuple(inp[n][e:e + 1] for n in ("w_gate", "w_up", "w_down"))
                t1 = time.perf_counter()
                xp = O.gather_rows(inp["x"], tok)
                G, U, H, Ov = O.ffn_forward_mx(xp, *w, one)
                d_o = gates[tok, slot][:, None] * np.asarray(inp["dy"][tok], dtype=np.float64)
                O.ffn_backward_mx(d_o, xp, *w, one, G, U, H)
                t_ffn += time.perf_counter() - t1
                n_e += 1
            e += 1
        # Token-level steps on the same share of tokens (values do not change
        # their cost): combine, combine backward and dispatch backward.
        Ts = max(1, T * n_e // E)
        sub_rows = row_of_slot[:Ts]
        rr = np.arange(Ts * k).reshape(Ts, k)
        o_sub = np.asarray(inp["x"][np.repeat(np.arange(Ts), k)], dtype=np.float64)
        t1 = time.perf_counter()
        O.combine(o_sub, gates[:Ts], rr)
        O.combine_backward(inp["dy"][:Ts], o_sub, gates[:Ts], rr)
        O.dispatch_backward(o_sub, rr)
        t_tok = time.perf_counter() - t1
        total = (t_ffn + t_tok) * E / n_e + t_plan
        return {"value": T / total, "unit": "tokens/s", "kind": "oracle", **host,
                "sample": f"fp64 MXFP8 oracle: FFN forward+backward of {n_e} whole experts' rows "
                          f"({int(counts[:e].max())} rows each; {t_ffn:.1f} s) plus combine, combine backward and "
                          f"dispatch backward on {Ts} tokens ({t_tok:.1f} s), scaled by E/{n_e} = {E / n_e:g}, "
                          f"plus the dispatch plan of all {T} tokens ({t_plan:.2f} s); {wl.name}, T={T}"}
    sub, Ts = inp, wl.T
    flops = 18.0 * wl.T * wl.k * wl.d * wl.f
    est_rate = 20e9 * threads  # fp64 flop/s, a first guess
    if flops / est_rate > budget_s:
        Ts = max(256, int(wl.T * budget_s * est_rate / flops) // 64 * 64)
        sub = make_inputs(wl.with_shape(T=Ts), 0)
    t0 = time.perf_counter()
    fwd = O.layer_forward(sub, wl.k)
    O.layer_backward(sub, fwd)
    dt = time.perf_counter() - t0
    what = "the whole workload" if Ts == wl.T else f"the first {Ts} tokens of the workload's inputs"
    return {"value": Ts / dt, "unit": "tokens/s", "kind": "oracle", **host,
            "sample": f"one fp64 forward+backward (oracle) of {what} ({wl.name}, T={wl.T}) on the host CPU, "
                      f"{dt:.1f} s"}


def load_traffic(name: str, dtype: str, mode: str):
    """The committed rocprofv3 counter summary of grouped-GEMM step `mode`
    (profiles/traffic_<name>.json: HBM bytes per launch, kernel names), if it
    was taken on the current sources of that kernel family; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        rec = json.load(fh)
    k = rec.get("gemm_kernels", {}).get(mode)
    if not k or k.get("kernel_source_hash") != kernel_source_hash(GEMM_SOURCES[dtype]):
        return None
    return k


def run_layer(wl, inp, args, M, torch, np):
    """Time one layer: warmup, a survey of the grouped-GEMM steps (one step
    each, kernel timer armed, untimed), the timed steps with the dominant
    GEMM step's launches bracketed by events, then cold-cache steps.
    Returns the figures of the JSON line for this layer."""
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16

    def dev(a, dtype=dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype)

    t = {n: dev(inp[n]) for n in ("x", "dy", "w_gate", "w_up", "w_down")}
    learned = wl.routing == "learned"
    if learned:
        t["w_router"] = dev(inp["w_router"])
    else:
        t["topk_idx"] = dev(inp["topk_idx"], torch.int32)
        t["topk_gate"] = dev(inp["topk_gate"], torch.float32)
    layer = M.MoELayer(wl.T, wl.d, wl.E, wl.k, wl.f, wl.dtype, learned_routing=learned, recompute=args.recompute)
    stream = torch.cuda.current_stream()

    def step(mark=None):
        if learned:
            layer.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"], w_router=t["w_router"], mark=mark)
        else:
            layer.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"], topk_idx=t["topk_idx"],
                          topk_gate=t["topk_gate"], mark=mark)
        layer.backward(t["dy"], mark=mark)

    def events(n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in ev:
            e.record(stream)  # creates the HIP event the library will re-record
        return ev

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Survey: each grouped-GEMM step's launch time, one untimed step each.
    mode_flops = gemm_mode_flops(wl, args.recompute)
    survey = {}
    for mi, mode in enumerate(GEMM_MODE_NAMES):
        st, sp = events(4), events(4)
        torch.cuda.synchronize()
        M.moe_kernel_timer(mi, st, sp)
        step()
        torch.cuda.synchronize()
        n = M.moe_kernel_timer_count()
        M.moe_kernel_timer(mi)
        ms = sum(a.elapsed_time(b) for a, b in zip(st[:n], sp[:n]))
        survey[mode] = {"launches_per_step": n, "ms_per_step": round(ms, 4),
                        "tflops": round(mode_flops[mode] / (ms * 1e-3) / 1e12, 1) if ms > 0 else None}
    dom = max(survey, key=lambda m: survey[m]["ms_per_step"])
    dom_i = GEMM_MODE_NAMES.index(dom)
    launches = survey[dom]["launches_per_step"]

    # Events on the stream the library launches on, one after each call; the
    # dominant GEMM step's launches bracketed by the library.
    marks = []  # per step: list of (name, event)

    def recorder(lst):
        def mark(name):
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(stream)
            lst.append((name, ev))
        return mark

    kst, ksp = events(launches * args.steps), events(launches * args.steps)
    torch.cuda.synchronize()
    M.moe_kernel_timer(dom_i, kst, ksp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        lst = []
        start = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        lst.append(("start", start))
        step(recorder(lst))
        marks.append(lst)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    nk = M.moe_kernel_timer_count()
    M.moe_kernel_timer(dom_i)
    kdur = [a.elapsed_time(b) for a, b in zip(kst[:nk], ksp[:nk])]

    per_call = {}
    for lst in marks:
        for (_, a), (name, b) in zip(lst[:-1], lst[1:]):
            per_call.setdefault(name, []).append(a.elapsed_time(b))
    avg_ms = {n: sum(v) / len(v) for n, v in per_call.items()}

    work = algorithmic_work(wl, args.recompute)
    gemm_ms = avg_ms["moe_grouped_ffn_fwd"] + avg_ms["moe_grouped_ffn_bwd"]
    gemm_flops = work["moe_grouped_ffn_fwd"]["flops"] + work["moe_grouped_ffn_bwd"]["flops"]
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    peak = {"f32": PEAK_F32_TFLOPS, "bf16": PEAK_BF16_TFLOPS, "mxfp8": PEAK_FP8_TFLOPS}[wl.dtype]
    calls = {}
    for n, ms in avg_ms.items():
        rec = {"ms": round(ms, 4)}
        if "flops" in work.get(n, {}):
            rec["tflops"] = round(work[n]["flops"] / (ms * 1e-3) / 1e12, 2)
        if "bytes" in work.get(n, {}):
            rec["gbs"] = round(work[n]["bytes"] / (ms * 1e-3) / 1e9, 1)
            rec["hbm_frac"] = round(rec["gbs"] / PEAK_HBM_GBS, 3)
        calls[n] = rec
    dc_names = [n for n in ("moe_dispatch", "moe_combine", "moe_combine_bwd", "moe_dispatch_bwd") if n in avg_ms]
    dc_bytes = sum(work[n]["bytes"] for n in dc_names)
    dc_ms = sum(avg_ms[n] for n in dc_names)

    # Against the combined roofline max(flops / MFMA peak, compulsory bytes /
    # HBM peak) of the two FFN calls (bf16 and fp32 layers: the MXFP8 calls
    # also quantise, which this count does not model).
    gemm_roof = None
    if wl.dtype != "mxfp8":
        gbytes = gemm_compulsory_bytes(wl)
        floor_ms = max(gemm_flops / (peak * 1e12), gbytes / (PEAK_HBM_GBS * 1e9)) * 1e3
        gemm_roof = {"compulsory_bytes": gbytes, "floor_ms": round(floor_ms, 4),
                     "bound": "mfma" if gemm_flops / (peak * 1e12) >= gbytes / (PEAK_HBM_GBS * 1e9) else "hbm",
                     "frac": round(floor_ms / gemm_ms, 4)}
    # The dominant kernel: algorithmic flops per launch (the step's flops
    # over its launches per step) / the average launch duration over the
    # timed region.
    flops_per_launch = mode_flops[dom] / launches
    avg_launch_ms = sum(kdur) / len(kdur)
    achieved = flops_per_launch / (avg_launch_ms * 1e-3) / 1e12
    # Counters were taken without recompute; an MXFP8 shape run on the bf16
    # path has its own file.
    from moe_inputs import WORKLOADS
    tname = wl.name if wl.dtype == WORKLOADS[wl.name].dtype else f"{wl.name}_as_{wl.dtype}"
    trec = None if args.recompute else load_traffic(tname, wl.dtype, dom)
    kname = trec["kernel"] if trec else {"mxfp8": "gg_mx_kernel / gg_mx_stream_kernel",
                                         "bf16": "gg_bf16_kernel / gg_bf16_stream_kernel",
                                         "f32": "grouped_gemm_kernel"}[wl.dtype]
    roofline = {"kernel": f"{kname} ({dom}: {launches} launch(es) per step)", "bound": "mfma",
                "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4),
                "traffic": trec["hbm_bytes_per_launch"] if trec else None,
                "flops_per_launch": flops_per_launch, "avg_launch_ms": round(avg_launch_ms, 4),
                "launches_timed": len(kdur)}
    ms_per_step = elapsed / args.steps * 1e3
    res = {
        "value": round(wl.T * args.steps / elapsed, 1), "ms_per_step": round(ms_per_step, 4),
        # bytes held between forward and backward beyond the inputs: the save
        # buffer (G, U, H unless recomputed; MXFP8 weight copies), xp (bf16
        # and fp32 layers), o, and for MXFP8 xp's two images.
        "saved_bytes": {"save": layer.save.numel(),
                        "xp": 0 if layer.xp is None else layer.xp.numel() * layer.xp.element_size(),
                        "o": layer.o.numel() * layer.o.element_size(),
                        "xp_mx": 0 if layer.xp_mx is None else layer.xp_mx.numel()},
        "grouped_gemm": {"tflops": round(gemm_tflops, 1), "frac_of_peak": round(gemm_tflops / peak, 4),
                         "peak_tflops": peak, "ms": round(gemm_ms, 4), "combined_roofline": gemm_roof,
                         "steps": survey},
        "dispatch_combine": {"gbs": round(dc_bytes / (dc_ms * 1e-3) / 1e9, 1),
                             "frac_of_hbm": round(dc_bytes / (dc_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "ms": round(dc_ms, 4)},
        "calls": calls,
        "roofline": roofline,
    }
    # Expert-load diagnostics of the last step's routing (moe_load_stats, after
    # the timed region).
    stats = layer.load_stats().cpu().tolist()
    res["expert_load"] = {n: round(v, 4) for n, v in zip(M.LOAD_STATS, stats)}
    # Cold caches: before each of K further steps a 1 GiB fill (untimed)
    # evicts the 256 MB MALL and the L2s; the step is timed by events around
    # it alone. The timed region above runs with the caches as the previous
    # step left them (warm).
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cold = []
    for _ in range(args.steps):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        cold.append((a, b))
    torch.cuda.synchronize()
    cold_ms = sorted(a.elapsed_time(b) for a, b in cold)
    med = cold_ms[len(cold_ms) // 2]
    res["cold_cache"] = {"ms_per_step_median": round(med, 4), "tokens_per_s": round(wl.T / (med * 1e-3), 1),
                         "flush_bytes": 1 << 30}
    del flush, layer, t
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mxfp8_balanced")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-twin", action="store_true",
                    help="MXFP8 workloads: skip the bf16 run of the same shape")
    ap.add_argument("--as-bf16", action="store_true",
                    help="run an MXFP8 workload's shape on the bf16 path only")
    ap.add_argument("--recompute", action="store_true",
                    help="activation recompute: save no G, U, H; the backward recomputes them")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB mebibytes (to scale HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import routing_grouped_gemm_softmax_amd as M
    from moe_inputs import WORKLOADS, make_inputs

    M.load()  # fails loudly if libmoe.so is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        # A plain device copy of known size: scales the HBM counters, and its
        # rate is the practical read+write bandwidth the copy kernels face.
        n = args.copy_calibration << 20
        a = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"copy_calibration_bytes": n, "copies": args.steps + 1, "ms_per_copy": round(ms, 4),
                          "read_plus_write_gbs": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return
    wl = WORKLOADS[args.workload]
    if args.as_bf16:
        wl = wl.with_shape(dtype="bf16")
    inp = make_inputs(wl, 0)
    res = run_layer(wl, inp, args, M, torch, np)
    out = {
        "metric": "MoE layer fwd+bwd tokens/s and grouped-GEMM TFLOP/s (% MFMA peak), 1 GPU",
        "value": res.pop("value"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": dict(wl.describe(), parallelism="none (1 GPU)",
                       **({"recompute": True} if args.recompute else {})),
    }
    out.update(res)
    if wl.dtype == "mxfp8" and not args.no_twin:
        # The bf16 path of the same shape and inputs (bf16 values), for the
        # MXFP8/bf16 ratio; its own timed steps, after the MXFP8 layer's.
        tw = run_layer(wl.with_shape(dtype="bf16"), inp, args, M, torch, np)
        out["bf16_twin"] = {"value": tw["value"], "unit": "tokens/s", "ms_per_step": tw["ms_per_step"],
                            "grouped_gemm": {k: tw["grouped_gemm"][k] for k in ("tflops", "frac_of_peak", "ms",
                                                                                "peak_tflops", "steps")},
                            "dispatch_combine": tw["dispatch_combine"], "calls": tw["calls"],
                            "roofline": tw["roofline"], "cold_cache": tw["cold_cache"]}
        out["mxfp8_over_bf16"] = round(out["value"] / tw["value"], 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
