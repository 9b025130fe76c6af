#!/usr/bin/env python3
"""Benchmark of the MSDA core operator on one MI355X: forward + backward per step.

Workload (the encoder-scale configuration): B=2, Q=S=22223 queries (one per pixel
of a 100x167, 50x84, 25x42, 13x21 pyramid, i.e. an ~800x1333 input at strides
8-64), M=8 heads, D=32, L=4 levels, K=4 points, fp32, offsets N(0, 2 px),
softmax weights; synthetic, seeded (workloads.py).

A step is one msda_forward (the library picks the schedule: at these sizes the
LDS-window gather; `--gather binned` times msda_forward_binned instead) plus one
msda_backward (grad_value, grad_sampling_locations, grad_attention_weights;
destination-binned by default) over one batch of inputs that is already
resident in HBM.  `--method softmax` times the "softmax" method instead
(msda_forward_softmax + msda_backward_softmax on raw logits).  `--rotate R` cycles over R independently generated
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


def bytes_model(wl: workloads.Workload, scatter: str = "binned") -> dict:
    """Algorithmic (compulsory) HBM bytes per launch of each kernel, each tensor once.

    For the encoder workloads every pyramid pixel is the reference point of a
    query and offsets are a few pixels, so every value row is touched and the
    whole value tensor counts.  Per-sample figures: loc 2 elements, attn 1
    element.  Only the operator's own tensors are compulsory: the forward reads
    value, loc and attn and writes out (28 B per sample at the encoder size);
    the backward reads value, loc, attn and grad_out and writes grad_value,
    grad_loc and grad_attn (48 B per sample).  The binned backward's dominant
    kernel (bin_tile) is charged the whole backward's compulsory bytes; the
    16-byte records it and the scatter pass exchange through the workspace are
    reported apart ("bin_records"), as are the fill kernel's bytes (the
    grad_value accumulator on the atomic path; on the binned path the per-bin
    counters: 8 stripes, one 64-byte line each, per 8x8 tile of every batch and
    head, plus 24 bytes per 256 bins of plan status)."""
    elt = 4 if wl.dtype == "fp32" else 2
    B, S, Q, M, D, L, K = wl.B, wl.S, wl.num_queries, wl.M, wl.D, wl.L, wl.K
    n = B * Q * M * L * K
    value = B * S * M * D * elt
    loc = n * 2 * elt
    attn = n * elt
    out = B * Q * M * D * elt
    recs = n * 16
    nbins = B * M * sum(-(-h // 8) * -(-w // 8) for h, w in wl.shapes)
    counters = nbins * 8 * 64 + -(-nbins // 256) * 24
    hq = B * Q * M
    return {
        "samples": n,
        # forward: gather value, read loc / attn, write out
        "fwd": value + loc + attn + out,
        # query-binned forward: the key reads the K finest-level points of every
        # head-query and writes a 4-byte key; the scatter reads the keys and writes
        # 4-byte sorted indices; the tile pass reads them once more
        "fwd_count": hq * K * 2 * elt + hq * 4,
        "fwd_scatter": hq * 8,
        "fwd_tile": value + loc + attn + out + hq * 4,
        # softmax method: the fused forward reads logits in place of weights; the
        # backward's row passes read logits and write weights, then read logits and
        # grad_attn and write grad_logits
        "fwd_softmax": value + loc + attn + out,
        "softmax_rows": 2 * attn,
        "softmax_grad_rows": 3 * attn,
        # the backward's compulsory bytes: value, loc, attn, grad_out read; grad_value,
        # grad_loc, grad_attn written
        "bwd": value + loc + attn + out + value + loc + attn,
        "bwd_atomic": value + loc + attn + out + value + loc + attn,
        "zero": value if scatter == "atomic" else counters,
        # binned passes (bin_tile: the whole backward's compulsory bytes)
        "bin_count": loc,
        "bin_scatter": loc + attn,
        "bin_tile": value + loc + attn + out + value + loc + attn,
        "bin_merge": 0,
        "bin_plan": 0,
        "bin_records": recs,
        "corner_rows": n * 4 * D * elt,
        "value": value,
    }


KERNEL_SOURCES = ("msda_kernels.hip", "msda_binned.hip", "msda_fwd_binned.hip", "msda_device.h",
                  "msda_launch.h")


def kernel_source_digest() -> str:
    """Digest of the operator's kernel sources: measured traffic is void once they change."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scale_deformable_attention_msda_amd", "csrc")
    for name in KERNEL_SOURCES:
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def read_counters(path: str, workload: str, scatter: str) -> dict:
    """Per-kernel counter figures from a profiles/ summary: {kernel: {"traffic": bytes per
    launch, "l2_hit": fraction}}, or {} when the summary is missing or was taken from other
    kernel sources than the current ones.

    The summary holds lines `sources: <digest>`, `traffic <workload>/<scatter>/<kernel>: <bytes>`
    and `l2hit <workload>/<scatter>/<kernel>: <fraction>`."""
    if not os.path.exists(path):
        return {}
    digest, out = None, {}
    for line in open(path):
        line = line.strip()
        if line.startswith("sources:"):
            digest = line.split(":", 1)[1].strip()
            continue
        for tag, field, conv in (("traffic", "traffic", lambda v: int(float(v))),
                                 ("l2hit", "l2_hit", float)):
            pre = f"{tag} {workload}/{scatter}/"
            if line.startswith(pre) and ":" in line:
                kernel, val = line[len(pre):].split(":", 1)
                try:
                    out.setdefault(kernel.strip(), {})[field] = conv(val.split()[0])
                except (ValueError, IndexError):
                    pass
    return out if digest == kernel_source_digest() else {}


# stated tolerances (rtol, atol): forward and backward fp32, bf16, fp16
TOLERANCES = {"fp32": {"out": (1e-5, 1e-6), "grad": (1e-4, 1e-5)},
              "bf16": {"out": (2e-2, 2e-2), "grad": (2e-2, 2e-2)},
              "fp16": {"out": (2.5e-3, 2.5e-3), "grad": (2.5e-3, 2.5e-3)}}


def parity_report(gpu: dict, ref: dict, dtype: str) -> dict:
    """Largest errors of the GPU outputs against the oracle's, and the count of elements
    outside the stated tolerance (|gpu - oracle| <= atol + rtol |oracle|)."""
    rep = {}
    for name, want in ref.items():
        got = np.asarray(gpu[name], dtype=np.float64).ravel()
        want = np.asarray(want, dtype=np.float64).ravel()
        rtol, atol = TOLERANCES[dtype]["out" if name == "out" else "grad"]
        err = np.abs(got - want)
        bad = ~(err <= atol + rtol * np.abs(want))
        rel = err / np.maximum(np.abs(want), atol)
        rep[name] = {"max_abs_err": float(np.max(err)), "max_rel_err": float(np.max(rel)),
                     "outside_tol": int(bad.sum()), "elements": int(got.size),
                     "rtol": rtol, "atol": atol}
    return rep


def cpu_baseline(x: dict, budget_s: float = 10.0, gpu: dict | None = None) -> dict:
    """The oracle timed on the host over the whole workload; with `gpu` (the library's
    outputs for the same inputs) the oracle's results also give the run's parity figures."""
    import oracle

    orc = oracle.default()
    args = (x["value"], x["spatial_shapes"], x["level_start_index"], x["sampling_locations"],
            x["attention_weights"])
    times = []
    t_end = time.perf_counter() + budget_s
    res = None
    while not times or (time.perf_counter() < t_end and len(times) < 20):
        t0 = time.perf_counter()
        out = orc.forward(*args)
        grads = orc.backward(*args, x["grad_out"])
        times.append(time.perf_counter() - t0)
        res = (out, grads)
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    base = {"value": float(np.mean(times)) * 1e6, "unit": "us/call", "cores": orc.threads(),
            "kind": "oracle",
            "sample": f"the whole workload, fp64 oracle forward+backward, {len(times)} calls "
                      f"(host: {cpu}, {os.cpu_count()} logical CPUs, {platform.machine()})"}
    if gpu is not None:
        out, (gv, gl, ga) = res
        base["parity"] = parity_report(gpu, {"out": out, "grad_value": gv, "grad_loc": gl,
                                             "grad_attn": ga}, x["dtype"])
    return base


CLOCK_GHZ = 2.4  # MI355X peak engine clock
CUS = 256


def microbenchmarks(msda, dev, stream) -> dict:
    """Ceilings of the memory paths on this GPU, from the library's microbenchmarks
    (include/msda_bench.h): streaming read and copy of 1 GiB, fp32 and packed-bf16 global
    atomics over whole 128-byte rows (random over 256 MiB, and piled on a 64 KiB hot set),
    gathers of random 128-byte rows from the vector L1 (16 KiB span), an L2-sized span
    (2 MiB), a value-tensor-sized span (64 MiB, L2 / MALL) and HBM (1 GiB), from LDS, and
    LDS fp32 atomics.  B/clk/CU uses the 2.4 GHz peak clock and 256 CUs."""
    import torch

    buf = torch.empty(2 ** 30 + 2 ** 20, dtype=torch.uint8, device=dev)

    def run(kind, span=0, reps=10):
        ms, units = msda.msda_microbench_run(kind, buf, span=span, reps=reps, stream=stream)
        return units / (ms * 1e-3)

    r = {}
    r["read_gbps"] = round(run("read") / 1e9, 1)
    r["copy_gbps"] = round(run("copy") / 1e9, 1)
    r["atomic_f32_spread_gops"] = round(run("atomic_f32", 2 ** 28) / 1e9, 1)
    r["atomic_f32_hot_gops"] = round(run("atomic_f32", 2 ** 16) / 1e9, 1)
    r["atomic_pk_bf16_spread_gpairs"] = round(run("atomic_pk_bf16", 2 ** 28) / 1e9, 1)
    r["atomic_pk_bf16_hot_gpairs"] = round(run("atomic_pk_bf16", 2 ** 16) / 1e9, 1)
    per_clk = CUS * CLOCK_GHZ * 1e9
    for name, span in (("l1", 2 ** 14), ("l2", 2 ** 21), ("value_span", 2 ** 26), ("hbm", 2 ** 30)):
        bps = run("gather_global", span)
        r[f"gather_{name}_gbps"] = round(bps / 1e9, 1)
        r[f"gather_{name}_b_per_clk_cu"] = round(bps / per_clk, 1)
    bps = run("gather_lds")
    r["gather_lds_gbps"] = round(bps / 1e9, 1)
    r["gather_lds_b_per_clk_cu"] = round(bps / per_clk, 1)
    r["lds_atomic_f32_per_clk_cu"] = round(run("lds_atomic_f32") / per_clk, 3)
    r["how"] = ("msda_microbench_run (libmsda.so), mean of 10 launches after one warm-up; "
                "read / copy of 1 GiB (L2 and MALL hold 288 MB, so both stream from HBM); "
                "atomics: whole 128-byte rows per instruction, rows random over 256 MiB "
                "(spread) or 64 KiB (hot); gathers: 8 lanes x 16 B per random 128-byte row, "
                "8 rows in flight per lane, 4 FMAs per 16 B")
    del buf
    return r


def cpu_baseline_single_thread(workload_id: int, seed: int, budget_s: float = 30.0) -> dict | None:
    """The oracle on one host thread, in a child process (OMP_NUM_THREADS=1), on
    the same seeded inputs; None if the child fails or runs over its budget."""
    import subprocess

    code = (
        "import sys, time, json\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import workloads, oracle\n"
        f"x = workloads.make_inputs({workload_id}, seed={seed})\n"
        "a = (x['value'], x['spatial_shapes'], x['level_start_index'], x['sampling_locations'],"
        " x['attention_weights'])\n"
        "o = oracle.default()\n"
        "t0 = time.perf_counter(); o.forward(*a); o.backward(*a, x['grad_out'])\n"
        "print(json.dumps({'s': time.perf_counter() - t0, 'threads': o.threads()}))\n")
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=budget_s)
        j = json.loads(r.stdout.strip().splitlines()[-1])
    except Exception:  # noqa: BLE001 - a missing figure is reported as null
        return None
    return {"value": round(j["s"] * 1e6, 1), "unit": "us/call", "cores": j["threads"]}


def grid_sample_msda_softmax(value, spatial_shapes, level_start_index, sampling_locations,
                             attention_logits, spatial_shapes_host):
    """The softmax-method operator composed from torch ops alone, for comparison:
    torch.softmax over the L*K logits, then per level one
    F.grid_sample(align_corners=False, padding_mode="zeros") of that level's
    value map at grid = 2 * location - 1 (the equivalence chapter 1 of the
    msda-triton course states, section "Bilinear interpolation: reading between
    the pixels"), weighted and summed over levels and points.  Autograd provides
    its backward; every intermediate it saves is what the fused kernels avoid."""
    import torch
    import torch.nn.functional as F

    B, S, M, D = value.shape
    Q, L, K = sampling_locations.shape[1], sampling_locations.shape[3], sampling_locations.shape[4]
    a = torch.softmax(attention_logits.reshape(B, Q, M, L * K), dim=-1).view(B, Q, M, L, K)
    out = None
    start = 0
    for lvl in range(L):
        H, W = int(spatial_shapes_host[lvl][0]), int(spatial_shapes_host[lvl][1])
        vl = value[:, start:start + H * W].permute(0, 2, 3, 1).reshape(B * M, D, H, W)
        grid = (2.0 * sampling_locations[:, :, :, lvl] - 1.0).permute(0, 2, 1, 3, 4)
        s = F.grid_sample(vl, grid.reshape(B * M, Q, K, 2), mode="bilinear",
                          padding_mode="zeros", align_corners=False)        # (B*M, D, Q, K)
        w = a[:, :, :, lvl].permute(0, 2, 1, 3).reshape(B * M, 1, Q, K)
        part = (s * w).sum(-1)                                                 # (B*M, D, Q)
        out = part if out is None else out + part
        start += H * W
    return out.view(B, M, D, Q).permute(0, 3, 1, 2).reshape(B, Q, M * D)


def layer_comparison(wl: workloads.Workload, dev, steps: int = 5) -> dict:
    """A multi-scale deformable attention layer (projections around the operator,
    softmax method) at the workload's sizes, forward + backward: the library's
    kernels against the grid_sample composition.  Peak memory is the growth of
    torch's allocated bytes over one step beyond what is resident before it
    (parameters, inputs); time is the median of `steps` steps (HIP events)."""
    import torch

    from scale_deformable_attention_msda_amd.layer import MultiScaleDeformAttn

    B, Q, S, M, D, L, K = wl.B, wl.num_queries, wl.S, wl.M, wl.D, wl.L, wl.K
    C = M * D
    dt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[wl.dtype]
    gen = torch.Generator(device="cpu").manual_seed(workloads.BASE_SEED)
    query = torch.randn(B, Q, C, generator=gen).to(dev, dt)
    value = torch.randn(B, S, C, generator=gen).to(dev, dt)
    gout = torch.randn(B, Q, C, generator=gen).to(dev, dt)
    host = np.asarray(wl.shapes, dtype=np.int64).reshape(L, 2)
    shapes = torch.from_numpy(host).to(dev)
    starts = torch.from_numpy(workloads.level_start_index(wl.shapes)).to(dev)
    if wl.ref == "pixel_centres":
        ref = torch.from_numpy(workloads.pixel_centre_refs(wl.shapes)).to(dev, dt)
        ref = ref[None, :, None, :].expand(B, Q, L, 2).contiguous()
    else:
        ref = torch.rand(B, Q, 1, 2, generator=gen).to(dev, dt).expand(B, Q, L, 2).contiguous()
    res = {}
    for name, sampler, scatter in (("library", None, "binned"),
                                   ("library_atomic", None, "atomic"),
                                   ("grid_sample", grid_sample_msda_softmax, "binned")):
        torch.manual_seed(0)
        layer = MultiScaleDeformAttn(C, M, L, K, sampler=sampler, scatter=scatter).to(dev, dt)

        def one_step():
            layer.zero_grad(set_to_none=True)
            out = layer(query, ref, value, shapes, starts, host)
            out.backward(gout)

        for _ in range(2):
            one_step()
        torch.cuda.synchronize()
        layer.zero_grad(set_to_none=True)
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        one_step()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev) - base
        ts = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            one_step()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        res[name] = {"ms_per_step": round(float(np.median(ts)), 3),
                     "peak_mib": round(peak / 2 ** 20, 1)}
        del layer
        torch.cuda.empty_cache()
    for name in ("library", "library_atomic"):
        res[name]["peak_vs_grid_sample"] = round(res[name]["peak_mib"] /
                                                 res["grid_sample"]["peak_mib"], 4)
    res["how"] = (f"dim {C}, {M} heads, {L} levels, {K} points, B={B}, Q={Q}, S={S}, {wl.dtype}; "
                  "library = the layer on msda_forward_softmax / msda_backward_softmax (binned or "
                  "atomic scatter); grid_sample = the same layer on torch.softmax + F.grid_sample; "
                  "peak = torch max_memory_allocated growth over one forward + backward step; "
                  f"time = median of {steps} steps")
    return res


def graph_comparison(dev, wid: int = 1, n: int = 50) -> dict:
    """One forward + backward step at a small configuration (launch-bound): n steps
    enqueued back to back from Python, against n replays of the same step captured
    once in a HIP graph (torch.cuda.CUDAGraph).  Microseconds per step."""
    import torch

    import scale_deformable_attention_msda_amd as msda

    wl = workloads.WORKLOADS[wid]
    x = workloads.make_inputs(wid)
    dt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[wl.dtype]
    t = {k: torch.from_numpy(x[k]).to(dev, dt) for k in
         ("value", "sampling_locations", "attention_weights", "grad_out")}
    shapes = torch.from_numpy(x["spatial_shapes"]).to(dev)
    starts = torch.from_numpy(x["level_start_index"]).to(dev)
    host = x["spatial_shapes"]
    ops = (t["value"], shapes, starts, t["sampling_locations"], t["attention_weights"])
    out, gv = torch.empty_like(t["grad_out"]), torch.empty_like(t["value"])
    gl, ga = torch.empty_like(t["sampling_locations"]), torch.empty_like(t["attention_weights"])
    dims = msda.MsdaDims(wl.B, wl.S, wl.M, wl.D, wl.L, wl.num_queries, wl.K)
    need = msda.msda_backward_workspace_bytes(dims, msda._DTYPES[dt], msda.MSDA_FP32,
                                              msda.MSDA_SCATTER_BINNED, host)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def step():
        msda.msda_forward(*ops, out=out)
        msda.msda_backward(*ops, t["grad_out"], grad_value=gv, grad_loc=gl, grad_attn=ga,
                           spatial_shapes_host=host, workspace=ws)

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    eager_us = timed(step)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    graph_us = timed(g.replay)
    return {"workload": f"{wl.name}: B={wl.B} Q={wl.num_queries} S={wl.S} M={wl.M} D={wl.D} "
                        f"L={wl.L} K={wl.K} {wl.dtype}",
            "eager_us": round(eager_us, 2), "graph_us": round(graph_us, 2),
            "how": f"{n} forward + binned backward steps enqueued back to back, eager from "
                   "Python against replays of one captured step"}


def need_f_plan(wl, dims, dcode, shapes_host) -> bool:
    """Whether the query-binned forward plans these sizes."""
    import scale_deformable_attention_msda_amd as msda

    try:
        return msda.msda_forward_binned_workspace_bytes(dims, dcode, shapes_host) > 0
    except ValueError:
        return False


def percentiles(xs) -> dict:
    a = np.sort(np.asarray(xs, dtype=np.float64))
    return {"p10": round(float(np.percentile(a, 10)), 3), "p50": round(float(np.percentile(a, 50)), 3),
            "p90": round(float(np.percentile(a, 90)), 3)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, help="workload id in workloads.py")
    ap.add_argument("--rotate", type=int, default=4, help="input batches cycled over")
    ap.add_argument("--scatter", default="binned", choices=["binned", "atomic"],
                    help="how the backward forms grad_value")
    ap.add_argument("--gather", default="direct", choices=["direct", "binned"],
                    help="forward schedule: msda_forward (direct gather) or msda_forward_binned")
    ap.add_argument("--reuse-order", action="store_true",
                    help="with --gather binned: sort once (in the warm-up) and reuse that query "
                         "order (msda_forward_binned_reuse)")
    ap.add_argument("--method", default="default", choices=["default", "softmax"],
                    help="attention weights as given, or softmax of raw logits in the operator")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the warm / cold regimes and the bandwidth microbenchmarks")
    ap.add_argument("--traffic-file", default=os.path.join(ROOT, "profiles", "traffic_encoder.txt"),
                    help="measured HBM bytes per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the operator has no "
              "multi-GPU path; a sharded run would give each GPU its own batch slice.",
              file=sys.stderr)
        return 2

    import torch

    import scale_deformable_attention_msda_amd as msda

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    if args.calibrate_copy:
        # a copy of known size: FETCH_SIZE / WRITE_SIZE of its kernel calibrate the counters
        n = 256 * 2 ** 20 // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "launches": 5}))
        return 0
    if args.method == "softmax" and args.gather != "direct":
        log("the softmax method runs on the direct gather only")
        return 2
    if args.reuse_order and args.gather != "binned":
        log("--reuse-order applies to --gather binned")
        return 2
    msda.load_library()
    wl = workloads.WORKLOADS[args.workload]
    dt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[wl.dtype]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    log(f"[bench] generating {args.rotate} input batch(es) of workload {wl.name}")
    host = [workloads.make_inputs(wl, seed=workloads.BASE_SEED + args.workload + 1000 * r)
            for r in range(args.rotate)]
    batches = []
    for x in host:
        t = {k: torch.from_numpy(x[k]).to(dev).to(dt) for k in
             ("value", "sampling_locations", "attention_weights", "attention_logits", "grad_out")}
        t["spatial_shapes"] = torch.from_numpy(x["spatial_shapes"]).to(dev)
        t["level_start_index"] = torch.from_numpy(x["level_start_index"]).to(dev)
        batches.append(t)
    t0 = batches[0]
    shapes_host = host[0]["spatial_shapes"]
    out = torch.empty_like(t0["grad_out"])
    gv = torch.empty_like(t0["value"])
    gl = torch.empty_like(t0["sampling_locations"])
    ga = torch.empty_like(t0["attention_weights"])
    dims = msda.MsdaDims(wl.B, wl.S, wl.M, wl.D, wl.L, wl.num_queries, wl.K)
    sc = msda.MSDA_SCATTER_BINNED if args.scatter == "binned" else msda.MSDA_SCATTER_ATOMIC
    dcode = msda._DTYPES[dt]
    need_b = msda.msda_backward_workspace_bytes(dims, dcode, msda.MSDA_FP32, sc, shapes_host)
    need_s = msda.msda_backward_softmax_workspace_bytes(dims, dcode, msda.MSDA_FP32, sc,
                                                        shapes_host)
    need_f = (msda.msda_forward_binned_workspace_bytes(dims, dcode, shapes_host)
              if args.gather == "binned" else 0)
    # one workspace serves both calls: they run one after the other on one stream
    # (with --reuse-order the forward keeps its own, which holds the order)
    need = max(need_b, need_s) if args.reuse_order else max(need_b, need_f, need_s)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(max(need_f, 1), dtype=torch.uint8, device=dev) if args.reuse_order else ws
    log(f"[bench] gather={args.gather} (workspace {need_f / 2**20:.1f} MiB), "
        f"scatter={args.scatter} (workspace {need_b / 2**20:.1f} MiB)")

    def ops(t):
        return (t["value"], t["spatial_shapes"], t["level_start_index"], t["sampling_locations"],
                t["attention_weights"])

    def ops_softmax(t):
        return ops(t)[:4] + (t["attention_logits"],)

    n_fwd_calls = [0]

    def fwd_plain(t):
        # with --reuse-order, the first call sorts and every later one reuses its order
        reuse = args.reuse_order and n_fwd_calls[0] > 0
        n_fwd_calls[0] += 1
        msda.msda_forward(*ops(t), out=out, stream=stream, gather=args.gather,
                          spatial_shapes_host=shapes_host, workspace=ws_f, reuse_order=reuse)

    def bwd_plain(t):
        msda.msda_backward(*ops(t), t["grad_out"], grad_value=gv, grad_loc=gl, grad_attn=ga,
                           scatter=args.scatter, spatial_shapes_host=shapes_host,
                           workspace=ws, stream=stream)

    def fwd_softmax(t):
        msda.msda_forward_softmax(*ops_softmax(t), out=out, stream=stream)

    def bwd_softmax(t):
        msda.msda_backward_softmax(*ops_softmax(t), t["grad_out"], grad_value=gv, grad_loc=gl,
                                   grad_logits=ga, scatter=args.scatter,
                                   spatial_shapes_host=shapes_host, workspace=ws, stream=stream)

    def step(i):
        t = batches[i % len(batches)]
        if args.method == "softmax":
            fwd_softmax(t)
            bwd_softmax(t)
        else:
            fwd_plain(t)
            bwd_plain(t)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    bm = bytes_model(wl, args.scatter)

    # kernel breakdown: a pass of its own, outside the timed region, with every
    # library kernel bracketed by HIP events on `stream`
    n_prof = 20
    msda.msda_profile_select(None)
    msda.msda_profile_start(64 * n_prof)
    for i in range(n_prof):
        step(i)
    torch.cuda.synchronize()
    per_kernel = {}
    for name, ms in msda.msda_profile_stop(64 * n_prof):
        per_kernel.setdefault(name, []).append(ms)
    kernels = {}
    for name, v in per_kernel.items():
        us = float(np.mean(v)) * 1e3
        nbytes = bm.get(name, 0)
        kernels[name] = {"us": round(us, 3), "launches_per_step": len(v) / n_prof,
                         "alg_bytes": nbytes,
                         "gbps": round(nbytes / (us * 1e-6) / 1e9, 1) if nbytes else None}
    dom_name = max(kernels, key=lambda n: kernels[n]["us"] * kernels[n]["launches_per_step"])

    # timed region: K steps; only the dominant kernel is bracketed by HIP events
    # (its live duration is the roofline's), so the other kernels run undisturbed
    msda.msda_profile_select(dom_name)
    msda.msda_profile_start(8 * args.steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    w0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    dom_ms = [ms for _, ms in msda.msda_profile_stop(8 * args.steps)]
    msda.msda_profile_select(None)
    step_us = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(args.steps)]

    def timed_steps(n, batch_of, before=None):
        """Per-step microseconds of n steps (events around each step only)."""
        out_us = []
        for i in range(n):
            if before is not None:
                before()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step(batch_of(i))
            e1.record(stream)
            e1.synchronize()
            out_us.append(e0.elapsed_time(e1) * 1e3)
        return out_us

    extras = {}
    if not args.no_extras:
        # regimes: warm = one input batch back to back (L2 / MALL resident);
        # cold = a 1 GiB buffer rewritten before every step (not timed), which
        # evicts the 8 x 4 MB L2 and the 256 MB MALL
        scratch = torch.empty(2 ** 28, dtype=torch.float32, device=dev)
        warm = timed_steps(20, lambda i: 0)
        cold = timed_steps(20, lambda i: 0, before=lambda: scratch.fill_(1.0))
        extras["regimes"] = {"rotate": dict(percentiles(step_us), steps=args.steps,
                                            batches=args.rotate),
                             "warm": dict(percentiles(warm), steps=20),
                             "cold": dict(percentiles(cold), steps=20)}
        # per-kernel durations with L2 and MALL evicted before every step
        msda.msda_profile_select(None)
        msda.msda_profile_start(64 * 10)
        for i in range(10):
            scratch.fill_(1.0)
            step(i)
        torch.cuda.synchronize()
        cold_k = {}
        for name, ms in msda.msda_profile_stop(64 * 10):
            cold_k.setdefault(name, []).append(ms)
        extras["regimes"]["cold"]["kernels_us"] = {n: round(float(np.mean(v)) * 1e3, 3)
                                                   for n, v in cold_k.items()}
        del scratch

        # what this GPU's memory paths reach (the library's own microbenchmarks)
        log("[bench] memory-path microbenchmarks")
        extras["achievable"] = microbenchmarks(msda, dev, stream)

        # the softmax method, fused against unfused: each call alone, over the rotated batches
        def call_us(fn, n=20, bl=None):
            bl = batches if bl is None else bl
            ts = []
            for i in range(n):
                t = bl[i % len(bl)]
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn(t)
                e1.record(stream)
                e1.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            return round(float(np.median(ts)), 2)

        LK = wl.L * wl.K

        def fwd_unfused(t):
            z = t["attention_logits"]
            a = torch.softmax(z.view(-1, LK), dim=-1).view(z.shape)
            msda.msda_forward(*ops(t)[:4], a, out=out, stream=stream)

        if wl.ref == "pixel_centres" and args.gather == "direct":
            # dispatch order: the kernels take head-queries in memory order, so
            # permuting the query axis of the inputs reorders the dispatch
            log("[bench] query dispatch orders")
            orders = {}
            for kind in ("linear", "morton", "hilbert"):
                perm = torch.from_numpy(workloads.query_order(wl.shapes, kind)).to(dev)
                pb = [dict(t, **{k: t[k][:, perm].contiguous() for k in
                                 ("sampling_locations", "attention_weights", "grad_out")})
                      for t in batches]
                orders[kind] = {"fwd_us": call_us(fwd_plain, bl=pb),
                                "step_us": call_us(lambda t: (fwd_plain(t), bwd_plain(t)), bl=pb)}
                del pb
            orders["how"] = ("queries of each level visited in raster, Z (Morton) or Hilbert "
                             "order, levels in sequence; median of 20 single forward calls and "
                             "of 20 forward + backward steps over the rotated batches")
            extras["query_order"] = orders

        # the atomic scatter (the pages' design) against what device-scope fp32
        # atomics reach on this GPU: the atomic_f32 microbenchmark (whole 128-byte
        # rows per instruction, the best pattern measured)
        log("[bench] atomic scatter and the atomic-add ceiling")
        adds = bm["samples"] * 4 * wl.D
        t0 = batches[0]
        gv_a = torch.empty_like(t0["value"])

        def bwd_atomic(t):
            msda.msda_backward(*ops(t), t["grad_out"], grad_value=gv_a, grad_loc=gl, grad_attn=ga,
                               scatter="atomic", stream=stream)

        atomic_us = call_us(bwd_atomic, n=5)
        ceil = extras["achievable"]["atomic_f32_spread_gops"] * 1e9
        extras["atomic_scatter"] = {
            "bwd_us": atomic_us,
            "element_adds": adds,
            "adds_per_s": round(adds / (atomic_us * 1e-6), 1),
            "ceiling_adds_per_s": round(ceil, 1),
            "frac_of_ceiling": round(adds / (atomic_us * 1e-6) / ceil, 4),
            "how": "msda_backward with the atomic scatter (fp32 atomics into grad_value, or into "
                   "an fp32 workspace then a cast for half-precision data), median of 5 calls; "
                   "ceiling = the atomic_f32 microbenchmark (whole 128-byte rows, random over "
                   "256 MiB)"}
        if wl.dtype != "fp32":
            # the same scatter with the data type as accumulator: packed two-element
            # atomics straight into grad_value instead of an fp32 workspace and a cast
            log("[bench] atomic scatter with the packed half-precision accumulator")
            gv_p = torch.empty_like(t0["value"])

            def bwd_packed(t):
                msda.msda_backward(*ops(t), t["grad_out"], grad_value=gv_p, grad_loc=gl,
                                   grad_attn=ga, accum_dtype=t0["value"].dtype,
                                   scatter="atomic", stream=stream)

            packed_us = call_us(bwd_packed, n=5)
            bwd_atomic(t0)
            bwd_packed(t0)
            torch.cuda.synchronize()
            ref = gv_a.double()
            rel_l2 = ((gv_p.double() - ref).norm() / ref.norm()).item()
            extras["atomic_scatter"]["packed_accumulator"] = {
                "bwd_us": packed_us,
                "pair_adds_per_s": round(adds / 2 / (packed_us * 1e-6), 1),
                "rel_l2_vs_fp32_accumulator": rel_l2,
                "how": f"msda_backward with the atomic scatter and accum_dtype = {wl.dtype} "
                       "(packed two-element atomics), median of 5 calls; rel_l2 = |gv_packed - "
                       "gv_fp32| / |gv_fp32| over grad_value on one batch"}
            del gv_p
        del gv_a

        log("[bench] HIP graph replay of a small (launch-bound) step")
        extras["graph"] = {"tiny": graph_comparison(dev, 0), "decoder": graph_comparison(dev, 1)}

        log("[bench] layer-level forward + backward against the grid_sample composition")
        extras["layer"] = layer_comparison(wl, dev)

        if args.gather == "direct" and need_f_plan(wl, dims, dcode, shapes_host):
            # the query-binned forward: sorting every call, or reusing the order that the
            # last sorted call left (taken from another input batch)
            log("[bench] query-binned forward, order sorted per call and reused")
            ws_o = torch.empty(msda.msda_forward_binned_workspace_bytes(dims, dcode, shapes_host),
                               dtype=torch.uint8, device=dev)

            def fwd_binned(t, reuse):
                msda.msda_forward(*ops(t), out=out, stream=stream, gather="binned",
                                  spatial_shapes_host=shapes_host, workspace=ws_o,
                                  reuse_order=reuse)

            extras["binned_forward"] = {
                "direct_us": call_us(fwd_plain),
                "binned_us": call_us(lambda t: fwd_binned(t, False)),
                "binned_reuse_us": call_us(lambda t: fwd_binned(t, True)),
                "how": "median of 20 single calls over the rotated batches; binned = "
                       "msda_forward_binned (sort + tile passes); reuse = "
                       "msda_forward_binned_reuse on the order the last sorted call left"}
            del ws_o

        if args.gather == "direct":
            extras["softmax_method"] = {
                "fwd_fused_us": call_us(fwd_softmax),
                "fwd_unfused_us": call_us(fwd_unfused),
                "fwd_plain_us": call_us(fwd_plain),
                "bwd_softmax_us": call_us(bwd_softmax),
                "bwd_plain_us": call_us(bwd_plain),
                "how": "median of 20 single calls over the rotated batches; unfused = "
                       "torch.softmax over the L*K logits, then msda_forward; plain = "
                       "msda_forward / msda_backward on given weights"}

    is_fwd = lambda n: n == "fwd" or n.startswith("fwd_")
    fwd_us = sum(k["us"] * k["launches_per_step"] for n, k in kernels.items() if is_fwd(n))
    bwd_us = sum(k["us"] * k["launches_per_step"] for n, k in kernels.items() if not is_fwd(n))
    ms_per_step = wall / args.steps * 1e3
    dom = kernels[dom_name]
    dom_us = float(np.mean(dom_ms)) * 1e3  # live, over the timed region
    dom["us_timed_region"] = round(dom_us, 3)
    achieved = dom["alg_bytes"] / (dom_us * 1e-6) / 1e9
    counters = read_counters(args.traffic_file, wl.name, args.scatter)
    for name, k in kernels.items():
        c = counters.get(name, {})
        if "traffic" in c:
            k["measured_bytes"] = c["traffic"]
            k["measured_gbps"] = round(c["traffic"] / (k["us"] * 1e-6) / 1e9, 1)
        if "l2_hit" in c:
            k["l2_hit"] = c["l2_hit"]
    traffic = counters.get(dom_name, {}).get("traffic")
    traffic_gbps = round(traffic / (dom_us * 1e-6) / 1e9, 1) if traffic else None
    step_bytes = bm["fwd"] + bm["bwd"]
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
        "dtype": {"fp32": "f32", "bf16": "bf16", "fp16": "f16"}[wl.dtype],
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={wl.B} Q=S={wl.num_queries} M={wl.M} D={wl.D} "
                               f"L={wl.L} (" + ", ".join(f"{h}x{w}" for h, w in wl.shapes) +
                               f") K={wl.K} {wl.dtype}, forward + backward",
                   "gather": args.gather, "scatter": args.scatter, "rotate": args.rotate,
                   "method": args.method},
        "fwd_us": round(fwd_us, 3),
        "bwd_us": round(bwd_us, 3),
        "kernels": kernels,
        "kernels_how": ("mean HIP-event duration per launch over a profiled pass of 20 steps "
                        "outside the timed region (every kernel bracketed); the timed region "
                        "brackets only the roofline kernel"),
        "queries_per_s": round(wl.B * wl.num_queries / (ms_per_step * 1e-3), 1),
        "fwd_hbm_gbps": round(bm["fwd"] / (fwd_us * 1e-6) / 1e9, 1),
        "fwd_hbm_frac": round(bm["fwd"] / (fwd_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        # the forward's target is 40% of the HBM peak: this is its fraction of that target
        "fwd_frac_of_target": round(bm["fwd"] / (fwd_us * 1e-6) / 1e9 / HBM_PEAK_GBPS / 0.40, 4),
        "bwd_hbm_gbps": round(bm["bwd"] / (bwd_us * 1e-6) / 1e9, 1),
        "bwd_hbm_frac": round(bm["bwd"] / (bwd_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "bytes_model": {"fwd": bm["fwd"], "bwd": bm["bwd"], "samples": bm["samples"],
                        "fwd_per_sample": round(bm["fwd"] / bm["samples"], 2),
                        "bwd_per_sample": round(bm["bwd"] / bm["samples"], 2),
                        "corner_rows": bm["corner_rows"], "bin_records": bm["bin_records"]},
        "step_hbm_gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": dom_name, "kernel_us": round(dom_us, 3),
                     "launches": len(dom_ms), "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "traffic_gbps": traffic_gbps},
    }
    res.update(extras)
    cold_k = extras.get("regimes", {}).get("cold", {}).get("kernels_us")
    if cold_k:
        # the HBM figures with L2 and MALL evicted before every step: inputs come from
        # HBM, not from a cache that still holds them (one launch of each kernel per step
        # on the default path; per-kernel means of the cold pass)
        c_fwd = sum(v for n, v in cold_k.items() if is_fwd(n))
        c_bwd = sum(v for n, v in cold_k.items() if not is_fwd(n))
        res["hbm_cold"] = {
            "step_p50_us": extras["regimes"]["cold"]["p50"],
            "fwd_us": round(c_fwd, 3), "bwd_us": round(c_bwd, 3),
            "fwd_frac": round(bm["fwd"] / (c_fwd * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "bwd_frac": round(bm["bwd"] / (c_bwd * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "how": "cold regime (a 1 GiB buffer rewritten before every step, not timed): "
                   "compulsory bytes over the kernels' mean HIP-event durations"}
        if dom_name in cold_k:
            res["hbm_cold"]["roofline_kernel_frac"] = round(
                dom["alg_bytes"] / (cold_k[dom_name] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
    if "achievable" in extras:
        ach = extras["achievable"]
        res["fwd_frac_of_read"] = round(bm["fwd"] / (fwd_us * 1e-6) / 1e9 / ach["read_gbps"], 4)
        # the forward's corner-row gather against the GPU's measured gather ceilings
        rate = bm["corner_rows"] / (fwd_us * 1e-6) / 1e9
        res["fwd_corner_gather"] = {
            "gbps": round(rate, 1),
            "b_per_clk_cu": round(rate * 1e9 / (CUS * CLOCK_GHZ * 1e9), 1),
            "frac_of_l1_gather": round(rate / ach["gather_l1_gbps"], 4),
            "frac_of_lds_gather": round(rate / ach["gather_lds_gbps"], 4),
            "us_at_l1_gather": round(bm["corner_rows"] / (ach["gather_l1_gbps"] * 1e9) * 1e6, 1),
            "us_at_lds_gather": round(bm["corner_rows"] / (ach["gather_lds_gbps"] * 1e9) * 1e6, 1)}
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        # the library's outputs for batch 0, compared with the oracle's in the same leg
        t = batches[0]
        if args.method == "softmax":
            gpu_out = None
        else:
            fwd_plain(t)
            bwd_plain(t)
            torch.cuda.synchronize()
            gpu_out = {"out": out.double().cpu().numpy(), "grad_value": gv.double().cpu().numpy(),
                       "grad_loc": gl.double().cpu().numpy(), "grad_attn": ga.double().cpu().numpy()}
        res["cpu_baseline"] = cpu_baseline(host[0], gpu=gpu_out)
        one = cpu_baseline_single_thread(args.workload, workloads.BASE_SEED + args.workload)
        if one is not None:
            res["cpu_baseline"]["single_thread"] = one
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
