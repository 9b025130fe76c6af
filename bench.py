#!/usr/bin/env python3
"""Benchmark of the MSDA core operator on one MI355X: forward + backward per step.

Workload (the encoder-scale configuration): B=2, Q=S=22223 queries (one per pixel
of a 100x167, 50x84, 25x42, 13x21 pyramid, i.e. an ~800x1333 input at strides
8-64), M=8 heads, D=32, L=4 levels, K=4 points, fp32, offsets N(0, 2 px),
softmax weights; synthetic, seeded (workloads.py).

A step is one msda_forward plus one msda_backward (grad_value by fp32 atomics,
grad_sampling_locations, grad_attention_weights) over one batch of inputs that
is already resident in HBM.  `--rotate R` cycles over R independently generated
input batches so that consecutive steps do not find their operands in the
L2 / MALL caches (R=1 times the warm, cache-resident regime).

Prints one JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "encoder-scale MSDA fwd+bwd µs/call and achieved HBM GB/s (% of peak)"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bytes_model(wl: workloads.Workload) -> dict:
    """Algorithmic (compulsory) HBM bytes per call, each tensor counted once.

    For the encoder workloads every pyramid pixel is the reference point of a
    query and offsets are a few pixels, so every value row is touched and the
    whole value tensor counts."""
    elt = 4 if wl.dtype == "fp32" else 2
    B, S, Q, M, D, L, K = wl.B, wl.S, wl.num_queries, wl.M, wl.D, wl.L, wl.K
    value = B * S * M * D * elt
    loc = B * Q * M * L * K * 2 * elt
    attn = B * Q * M * L * K * elt
    out = B * Q * M * D * elt
    return {
        "samples": B * Q * M * L * K,
        "fwd": value + loc + attn + out,
        # the scatter kernel: value, loc, attn, grad_out read once; grad_value,
        # grad_loc, grad_attn written once
        "bwd_kernel": value + loc + attn + out + value + loc + attn,
        "zero_fill": value,
        "value": value,
    }


def cpu_baseline(x: dict, budget_s: float = 10.0) -> dict:
    import oracle

    orc = oracle.default()
    args = (x["value"], x["spatial_shapes"], x["level_start_index"], x["sampling_locations"],
            x["attention_weights"])
    times = []
    t_end = time.perf_counter() + budget_s
    while not times or (time.perf_counter() < t_end and len(times) < 20):
        t0 = time.perf_counter()
        orc.forward(*args)
        orc.backward(*args, x["grad_out"])
        times.append(time.perf_counter() - t0)
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": float(np.mean(times)) * 1e6, "unit": "us/call", "cores": orc.threads(),
            "kind": "oracle",
            "sample": f"the whole workload, fp64 oracle forward+backward, {len(times)} calls "
                      f"(host: {cpu}, {os.cpu_count()} logical CPUs, {platform.machine()})"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, help="workload id in workloads.py")
    ap.add_argument("--rotate", type=int, default=4, help="input batches cycled over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): every box here has "
              "one GPU; see DESIGN.md for how the operator would shard.", file=sys.stderr)
        return 2

    import torch

    import scale_deformable_attention_msda_amd as msda

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    msda.load_library()
    wl = workloads.WORKLOADS[args.workload]
    dt = torch.float32 if wl.dtype == "fp32" else torch.bfloat16
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    log(f"[bench] generating {args.rotate} input batch(es) of workload {wl.name}")
    host = [workloads.make_inputs(wl, seed=workloads.BASE_SEED + args.workload + 1000 * r)
            for r in range(args.rotate)]
    batches = []
    for x in host:
        t = {k: torch.from_numpy(x[k]).to(dev).to(dt) for k in
             ("value", "sampling_locations", "attention_weights", "grad_out")}
        t["spatial_shapes"] = torch.from_numpy(x["spatial_shapes"]).to(dev)
        t["level_start_index"] = torch.from_numpy(x["level_start_index"]).to(dev)
        batches.append(t)
    t0 = batches[0]
    out = torch.empty_like(t0["grad_out"])
    gv = torch.empty_like(t0["value"])
    gl = torch.empty_like(t0["sampling_locations"])
    ga = torch.empty_like(t0["attention_weights"])
    ws = None
    dims = msda.MsdaDims(wl.B, wl.S, wl.M, wl.D, wl.L, wl.num_queries, wl.K)
    need = msda.msda_backward_workspace_bytes(dims, 0 if wl.dtype == "fp32" else 1, 0)
    if need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def ops(t):
        return (t["value"], t["spatial_shapes"], t["level_start_index"], t["sampling_locations"],
                t["attention_weights"])

    def step(i, ev=None):
        t = batches[i % len(batches)]
        if ev is not None:
            ev[0].record(stream)
        msda.msda_forward(*ops(t), out=out, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        msda.msda_backward(*ops(t), t["grad_out"], grad_value=gv, grad_loc=gl, grad_attn=ga,
                           workspace=ws, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    fwd_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    bwd_ms = np.array([e[1].elapsed_time(e[2]) for e in events])

    # zero-fill alone: a backward call with no queries only zero-fills grad_value
    fill_ms = []
    empty = {k: v for k, v in t0.items()}
    empty["sampling_locations"] = t0["sampling_locations"][:, :0]
    empty["attention_weights"] = t0["attention_weights"][:, :0]
    empty["grad_out"] = t0["grad_out"][:, :0]
    for i in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        msda.msda_backward(*ops(empty), empty["grad_out"], grad_value=gv,
                           grad_loc=gl[:, :0], grad_attn=ga[:, :0], workspace=ws, stream=stream)
        e[1].record(stream)
        fill_ms.append(e)
    torch.cuda.synchronize()
    fill_ms = np.array([e[0].elapsed_time(e[1]) for e in fill_ms])

    bm = bytes_model(wl)
    fwd_us = float(np.mean(fwd_ms)) * 1e3
    bwd_us = float(np.mean(bwd_ms)) * 1e3
    fill_us = float(np.mean(fill_ms)) * 1e3
    scatter_us = max(bwd_us - fill_us, 1e-3)
    ms_per_step = wall / args.steps * 1e3
    kernels = {
        "fwd": {"us": fwd_us, "bytes": bm["fwd"]},
        "bwd": {"us": scatter_us, "bytes": bm["bwd_kernel"]},
    }
    dom_name = max(kernels, key=lambda k: kernels[k]["us"])
    dom = kernels[dom_name]
    achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            rec = tj.get(f"{wl.name}/{dom_name}")
            if rec and rec.get("valid", False):
                traffic = rec["bytes_per_launch"]
        except (OSError, ValueError, KeyError):
            traffic = None
    fwdbwd_gbps = (bm["fwd"] + bm["bwd_kernel"] + bm["zero_fill"]) / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(ms_per_step * 1e3, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.dtype == "fp32" else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={wl.B} Q=S={wl.num_queries} M={wl.M} D={wl.D} "
                               f"L={wl.L} (" + ", ".join(f"{h}x{w}" for h, w in wl.shapes) +
                               f") K={wl.K} {wl.dtype}, fwd+bwd",
                   "rotate": args.rotate},
        "fwd_us": round(fwd_us, 3),
        "bwd_us": round(bwd_us, 3),
        "bwd_zero_fill_us": round(fill_us, 3),
        "bwd_kernel_us": round(scatter_us, 3),
        "queries_per_s": wl.B * wl.num_queries / (ms_per_step * 1e-3),
        "fwd_hbm_gbps": round(bm["fwd"] / (fwd_us * 1e-6) / 1e9, 1),
        "fwd_hbm_frac": round(bm["fwd"] / (fwd_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "bwd_hbm_gbps": round(bm["bwd_kernel"] / (scatter_us * 1e-6) / 1e9, 1),
        "fwdbwd_hbm_gbps": round(fwdbwd_gbps, 1),
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        res["cpu_baseline"] = cpu_baseline(host[0])
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
