"""Occupancy / tile-size sweep of the MSDA kernels on the encoder-scale workload.

The pages make occupancy a question to measure, not a goal: a tiling at low
occupancy beat one at high occupancy by a wide margin on their GPU ("Efficient
Multi-Scale Deformable Attention on GPUs", key findings and "Two heuristics
that do not apply"; the msda-triton course index, chapter 4).  This module
rebuilds the library with its tuning constants overridden (-D flags) and
measures every variant on one GPU:

  fwd_pipe     MSDA_FWD_PIPE        corner-row loads a forward lane keeps in flight (x4)
  fwd_block    MSDA_FWD_BLOCK       lanes per forward block (head-queries per block)
  win_pipe     MSDA_WIN_PIPE        samples in flight per lane, LDS-window forward
  win_blocks   MSDA_WIN_BLOCKS_PER_CU  LDS-window blocks per CU over the launch
  win_lds      MSDA_WIN_LDS_BLOCKS  LDS-window blocks sharing one CU's LDS
  bin_chunk    MSDA_BIN_CHUNK       samples per tile-kernel chunk (binned backward)
  bin_tile     MSDA_BIN_TILE        destination tile edge in pixels (binned backward)
  count_block  MSDA_COUNT_SAMPLES   samples per count / scatter block
  plan_block   MSDA_PLAN_BLOCK      bins per plan block (look-back over the blocks)

Per point it records the registers, LDS and waves per SIMD the compiler reports
for the kernels the constant touches, the per-kernel µs of a forward + binned
backward step (HIP events on the launch stream), and, with --counters, the
FETCH_SIZE / WRITE_SIZE / L2 hit rate rocprofv3 reads per launch (FETCH scaled
by the factor a plain copy of known size gives).  Every variant's outputs are
compared with those of the in-tree library on the same inputs (rtol 1e-5 /
atol 1e-6 forward, 1e-4 / 1e-5 backward; 1e-2 / 1e-3 for the 16-bit outputs of
the half-precision workloads, which `one --workload` also runs); that library
is the one the parity tests check against the oracle.

  python -m scale_deformable_attention_msda_amd.sweep build [--group G ...]   (CPU: compile)
  python -m scale_deformable_attention_msda_amd.sweep run [--group G ...] [--counters]
         [--out profiles/sweep_encoder.md]                                     (GPU)
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import shutil
import subprocess
import sys
import tempfile
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SWEEP_DIR = os.path.join(ROOT, "_build", "sweep")

GROUPS = {
    "fwd_pipe": [("pipe2", ["-DMSDA_FWD_PIPE=2"]), ("pipe4", ["-DMSDA_FWD_PIPE=4"]),
                 ("pipe8", ["-DMSDA_FWD_PIPE=8"])],
    "fwd_block": [("block128", ["-DMSDA_FWD_BLOCK=128"]), ("block256", ["-DMSDA_FWD_BLOCK=256"]),
                  ("block512", ["-DMSDA_FWD_BLOCK=512"]), ("block1024", ["-DMSDA_FWD_BLOCK=1024"])],
    "win_pipe": [("winpipe2", ["-DMSDA_WIN_PIPE=2"]), ("winpipe4", ["-DMSDA_WIN_PIPE=4"])],
    "win_lds": [("winlds1", ["-DMSDA_WIN_LDS_BLOCKS=1"]), ("winlds2", ["-DMSDA_WIN_LDS_BLOCKS=2"])],
    "win_blocks": [("winbpc1", ["-DMSDA_WIN_BLOCKS_PER_CU=1"]),
                   ("winbpc2", ["-DMSDA_WIN_BLOCKS_PER_CU=2"]),
                   ("winbpc4", ["-DMSDA_WIN_BLOCKS_PER_CU=4"])],
    "bin_chunk": [("chunk256", ["-DMSDA_BIN_CHUNK=256"]), ("chunk512", ["-DMSDA_BIN_CHUNK=512"]),
                  ("chunk1024", ["-DMSDA_BIN_CHUNK=1024"])],
    "bin_tile": [("tile7", ["-DMSDA_BIN_TILE=7"]), ("tile8", ["-DMSDA_BIN_TILE=8"]),
                 ("tile9", ["-DMSDA_BIN_TILE=9"]), ("tile10", ["-DMSDA_BIN_TILE=10"])],
    "count_block": [("count2048", ["-DMSDA_COUNT_SAMPLES=2048"]),
                    ("count4096", ["-DMSDA_COUNT_SAMPLES=4096"]),
                    ("count8192", ["-DMSDA_COUNT_SAMPLES=8192"])],
    "plan_block": [("plan64", ["-DMSDA_PLAN_BLOCK=64"]), ("plan128", ["-DMSDA_PLAN_BLOCK=128"]),
                   ("plan256", ["-DMSDA_PLAN_BLOCK=256"])],
}
# the kernels whose resources each group changes (names as the compiler reports them)
GROUP_KERNELS = {
    "fwd_pipe": ["fwd_kernel"], "fwd_block": ["fwd_kernel"], "win_pipe": ["fwd_win_kernel"],
    "win_blocks": ["fwd_win_kernel"], "win_lds": ["fwd_win_kernel"], "bin_chunk": ["tile_kernel"],
    "bin_tile": ["tile_kernel"], "count_block": ["count_kernel", "scatter_kernel"],
    "plan_block": ["plan_kernel"],
}
# forward schedule of the timed step per group: the direct-gather groups force
# the direct gather (the encoder takes the LDS-window schedule by default)
GROUP_SCHEDULE = {"fwd_pipe": "direct", "fwd_block": "direct"}
# library profile names of the kernels
PROFILE_NAME = {"fwd_kernel": "fwd", "fwd_win_kernel": "fwd", "tile_kernel": "bin_tile",
                "count_kernel": "bin_count",
                "scatter_kernel": "bin_scatter", "merge_kernel": "bin_merge",
                "plan_kernel": "bin_plan", "zero_kernel": "zero"}


def point_dir(name: str) -> str:
    return os.path.join(SWEEP_DIR, name)


# ------------------------------------------------------------------- build

def _resource_remarks(text: str) -> dict:
    """{mangled kernel: {"vgprs", "lds", "waves_per_simd", "scratch"}} from the
    compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        if cur is None:
            continue
        for key, pat in (("vgprs", r"remark:\s+VGPRs: (\d+)"), ("agprs", r"remark:\s+AGPRs: (\d+)"),
                         ("lds", r"remark:\s+LDS Size \[bytes/block\]: (\d+)"),
                         ("waves_per_simd", r"remark:\s+Occupancy \[waves/SIMD\]: (\d+)"),
                         ("scratch", r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")):
            m = re.search(pat, line)
            if m:
                cur[key] = int(m.group(1))
    return out


# fp32, D = 32, plain-method instantiations (Itanium mangling of the template arguments)
_INSTANCE = {
    "fwd_kernel": re.compile(r"\d+fwd_kernelIfLi32ELb0ELi(\d+)E"),
    "fwd_win_kernel": re.compile(r"\d+fwd_win_kernelIfLi32ELb0ELi(\d+)E"),
    "tile_kernel": re.compile(r"\d+tile_kernelIfLi32ELb1EE"),
    "count_kernel": re.compile(r"\d+count_kernelIfEE"),
    "scatter_kernel": re.compile(r"\d+scatter_kernelIfLb0EEE"),
    "plan_kernel": re.compile(r"\d+plan_kernelENS_7BinArgsE"),
}


def _relevant(remarks: dict, kernels: list[str]) -> dict:
    """Resources of the fp32, D = 32, plain-method instantiations of `kernels`."""
    res = {}
    for mangled, r in remarks.items():
        for base in kernels:
            m = _INSTANCE[base].search(mangled)
            if m:
                res[base + (f"<pipe {m.group(1)}>" if base.startswith("fwd") else "")] = r
    return res


def build_points(groups: list[str]) -> None:
    from scale_deformable_attention_msda_amd import build as b

    for g in groups:
        for name, flags in GROUPS[g]:
            d = point_dir(name)
            os.makedirs(d, exist_ok=True)
            log = []
            t0 = time.time()
            try:
                b.build(out=os.path.join(d, "libmsda.so"),
                        extra_flags=flags + ["-Rpass-analysis=kernel-resource-usage"], remarks=log)
                status = "built"
            except RuntimeError as e:
                status = "build failed: " + str(e).splitlines()[0][:200]
            res = _relevant(_resource_remarks("\n".join(log)), GROUP_KERNELS[g])
            json.dump({"group": g, "name": name, "flags": flags, "status": status,
                       "resources": res}, open(os.path.join(d, "point.json"), "w"), indent=1)
            print(f"[sweep build] {g}/{name} {flags}: {status} ({time.time() - t0:.0f} s) "
                  f"{json.dumps(res)}", flush=True)


# --------------------------------------------------------------------- one

def run_one(lib: str, workload: int, steps: int, ref_dir: str, write_ref: bool,
            schedule: str = "auto") -> dict:
    """Time one library variant on one GPU (child process) and compare its outputs."""
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import workloads
    import scale_deformable_attention_msda_amd as msda

    msda.load_library(lib)
    msda.msda_test_set_forward_schedule(schedule)
    wl = workloads.WORKLOADS[workload]
    dt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[wl.dtype]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    batches = []
    for r in range(2):
        x = workloads.make_inputs(wl, seed=workloads.BASE_SEED + workload + 1000 * r)
        t = {k: torch.from_numpy(x[k]).to(dev).to(dt) for k in
             ("value", "sampling_locations", "attention_weights", "grad_out")}
        t.update({k: torch.from_numpy(x[k]).to(dev) for k in ("spatial_shapes", "level_start_index")})
        batches.append(t)
    shapes_host = x["spatial_shapes"]
    t0 = batches[0]
    out = torch.empty_like(t0["grad_out"])
    gv, gl, ga = (torch.empty_like(t0["value"]), torch.empty_like(t0["sampling_locations"]),
                  torch.empty_like(t0["attention_weights"]))
    dims = msda.MsdaDims(wl.B, wl.S, wl.M, wl.D, wl.L, wl.num_queries, wl.K)
    mdt = {"fp32": msda.MSDA_FP32, "bf16": msda.MSDA_BF16, "fp16": msda.MSDA_FP16}[wl.dtype]
    need = msda.msda_backward_workspace_bytes(dims, mdt, msda.MSDA_FP32,
                                              msda.MSDA_SCATTER_BINNED, shapes_host)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step(t):
        ops = (t["value"], t["spatial_shapes"], t["level_start_index"], t["sampling_locations"],
               t["attention_weights"])
        msda.msda_forward(*ops, out=out, stream=stream)
        msda.msda_backward(*ops, t["grad_out"], grad_value=gv, grad_loc=gl, grad_attn=ga,
                           spatial_shapes_host=shapes_host, workspace=ws, stream=stream)

    for i in range(3):
        step(batches[i % 2])
    torch.cuda.synchronize()
    msda.msda_profile_select(None)
    msda.msda_profile_start(64 * steps)
    for i in range(steps):
        step(batches[i % 2])
    torch.cuda.synchronize()
    per = {}
    for name, ms in msda.msda_profile_stop(64 * steps):
        per.setdefault(name, []).append(ms * 1e3)
    us = {n: round(float(np.mean(v)) * len(v) / steps, 2) for n, v in per.items()}
    us["step"] = round(sum(us.values()), 2)
    # outputs of batch 0 against the in-tree library's
    step(t0)
    torch.cuda.synchronize()
    got = {"out": out, "grad_value": gv, "grad_loc": gl, "grad_attn": ga}
    parity = {}
    for k, v in got.items():
        a = v.float().cpu().numpy()
        path = os.path.join(ref_dir, k + ".npy")
        if write_ref:
            np.save(path, a)
            parity[k] = "reference"
            continue
        ref = np.load(path)
        if wl.dtype != "fp32":  # 16-bit outputs: a few units in the last place
            rtol, atol = 1e-2, 1e-3
        else:
            rtol, atol = (1e-5, 1e-6) if k == "out" else (1e-4, 1e-5)
        err = np.abs(a.astype(np.float64) - ref)
        bad = int((~(err <= atol + rtol * np.abs(ref.astype(np.float64)))).sum())
        parity[k] = {"max_abs": float(err.max()), "outside": bad}
    return {"us": us, "parity": parity}


# --------------------------------------------------------------------- run

def _counter_csv_rows(d: str) -> list[dict]:
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _kernel_base(name: str) -> str:
    """'void msda::(anonymous namespace)::tile_kernel<float, 32>(msda::BinArgs)' -> 'tile_kernel'."""
    base = name.replace("(anonymous namespace)", "").split("<")[0].split("(")[0]
    return base.split("::")[-1].strip()


def _profiled(lib: str, counters: list[str], out_dir: str, ref_dir: str, copy: bool = False,
              schedule: str = "auto") -> dict:
    """Mean counter values per kernel (library profile names) over one profiled child run."""
    d = tempfile.mkdtemp(prefix="sweep_pmc_", dir=out_dir)
    child = ([sys.executable, os.path.join(ROOT, "bench.py"), "--calibrate-copy"] if copy else
             [sys.executable, "-m", "scale_deformable_attention_msda_amd.sweep", "one", "--lib", lib,
              "--steps", "3", "--ref-dir", ref_dir, "--schedule", schedule])
    cmd = ["rocprofv3", "--pmc", *counters, "--output-format", "csv", "-d", d, "-o", "run", "--",
           *child]
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=300)
    rows = _counter_csv_rows(d)
    if r.returncode != 0 and not rows:
        raise RuntimeError(f"rocprofv3 failed ({r.returncode}): {r.stderr[-1500:]}")
    acc = {}
    for row in rows:
        base = _kernel_base(row.get("Kernel_Name", ""))
        key = "copy" if copy and "copy" in base.lower() else PROFILE_NAME.get(base)
        if key is None:
            continue
        per = acc.setdefault(key, {})
        # one row per (dispatch, counter): sum over a dispatch's rows, then average dispatches
        disp = per.setdefault(row.get("Counter_Name", ""), {})
        did = row.get("Dispatch_Id", str(len(disp)))
        disp[did] = disp.get(did, 0.0) + float(row.get("Counter_Value", 0) or 0)
    shutil.rmtree(d, ignore_errors=True)
    return {k: {c: sum(v.values()) / max(len(v), 1) for c, v in per.items()} for k, per in acc.items()}


def run_points(groups: list[str], counters: bool, out_md: str, steps: int) -> None:
    out_dir = tempfile.mkdtemp(prefix="msda_sweep_")  # reference outputs and counter runs
    ref_dir = tempfile.mkdtemp(prefix="sweep_ref_", dir=out_dir)
    default_lib = os.path.join(PKG, "libmsda.so")

    def child(lib, write_ref=False, schedule="auto"):
        cmd = [sys.executable, "-m", "scale_deformable_attention_msda_amd.sweep", "one", "--lib", lib,
               "--steps", str(steps), "--ref-dir", ref_dir, "--schedule", schedule] + \
              (["--write-ref"] if write_ref else [])
        r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=300)
        if r.returncode != 0:
            return {"error": r.stderr.strip().splitlines()[-1][:300] if r.stderr.strip() else
                    f"exit {r.returncode}"}
        return json.loads(r.stdout.strip().splitlines()[-1])

    print("[sweep] reference: the in-tree library", flush=True)
    ref = child(default_lib, write_ref=True)
    print(f"[sweep] default {json.dumps(ref)}", flush=True)
    scale = None
    if counters:
        f = _profiled("", ["FETCH_SIZE"], out_dir, ref_dir, copy=True).get("copy", {})
        w = _profiled("", ["WRITE_SIZE"], out_dir, ref_dir, copy=True).get("copy", {})
        nbytes = 256 * 2 ** 20
        if f.get("FETCH_SIZE") and w.get("WRITE_SIZE"):
            scale = (nbytes / (f["FETCH_SIZE"] * 1024), nbytes / (w["WRITE_SIZE"] * 1024))
        print(f"[sweep] copy calibration: FETCH x{scale[0] if scale else None}, "
              f"WRITE x{scale[1] if scale else None}", flush=True)
    results = []
    for g in groups:
        for name, flags in GROUPS[g]:
            d = point_dir(name)
            meta_path = os.path.join(d, "point.json")
            if not os.path.exists(meta_path):
                print(f"[sweep] {g}/{name}: not built", flush=True)
                continue
            meta = json.load(open(meta_path))
            lib = os.path.join(d, "libmsda.so")
            rec = dict(meta)
            sched = GROUP_SCHEDULE.get(g, "auto")
            rec["schedule"] = sched
            if meta["status"] == "built":
                rec.update(child(lib, schedule=sched))
                if counters and "error" not in rec:
                    try:
                        c1 = _profiled(lib, ["FETCH_SIZE"], out_dir, ref_dir, schedule=sched)
                        c2 = _profiled(lib, ["WRITE_SIZE", "TCC_HIT_sum", "TCC_MISS_sum"], out_dir,
                                       ref_dir, schedule=sched)
                        traffic = {}
                        for k in set(c1) | set(c2):
                            fkib = c1.get(k, {}).get("FETCH_SIZE")
                            wkib = c2.get(k, {}).get("WRITE_SIZE")
                            hit, miss = (c2.get(k, {}).get("TCC_HIT_sum"),
                                         c2.get(k, {}).get("TCC_MISS_sum"))
                            traffic[k] = {
                                "fetch_kib": fkib, "write_kib": wkib,
                                "bytes": (fkib * 1024 * scale[0] + wkib * 1024 * scale[1])
                                if (scale and fkib is not None and wkib is not None) else None,
                                "l2_hit": hit / (hit + miss) if hit is not None and miss else None}
                        rec["counters"] = traffic
                    except (RuntimeError, subprocess.TimeoutExpired) as e:
                        rec["counters_error"] = str(e)[:300]
            results.append(rec)
            print(f"[sweep] {g}/{name} {json.dumps(rec)}", flush=True)
    shutil.rmtree(out_dir, ignore_errors=True)
    write_summary(out_md, ref, results, scale, steps, counters)


def write_summary(path: str, ref: dict, results: list[dict], scale, steps: int, counters: bool):
    lines = ["# Tuning sweep: encoder workload, forward + binned backward", "",
             "Workload: B=2, Q=S=22223, M=8, D=32, L=4 (100x167, 50x84, 25x42, 13x21), K=4, fp32; "
             "one MI355X.", "",
             "Command (repository root on the GPU host; the variants are built beforehand on any "
             "host with `python -m scale_deformable_attention_msda_amd.sweep build`):", "",
             "    python -m scale_deformable_attention_msda_amd.sweep run"
             + (" --counters" if counters else "") + f" --steps {steps}", "",
             f"µs: mean HIP-event duration per step over {steps} steps (2 input batches "
             "alternating). Registers / LDS / waves per SIMD: the compiler's resource report for "
             "the fp32, D = 32 instantiation. Parity: every output against the in-tree library "
             "(whose tests check it against the oracle), elements outside rtol 1e-5 / atol 1e-6 (forward) and "
             "1e-4 / 1e-5 (backward)."]
    if counters:
        lines.append(
            "Counters: rocprofv3 `--pmc FETCH_SIZE` and `--pmc WRITE_SIZE TCC_HIT_sum TCC_MISS_sum` "
            "over a 3-step child run; bytes = FETCH_SIZE x %.3f + WRITE_SIZE x %.3f (the factors a "
            "plain 256 MiB copy gives), per launch; L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS)."
            % (scale if scale else (float("nan"), float("nan"))))
    lines += ["", f"In-tree library: {json.dumps(ref.get('us', ref))}", ""]
    lines.append("| group | point | flags | status | kernel resources (VGPRs / LDS B / waves per SIMD) "
                 "| fwd µs | tile µs | count µs | plan µs | scatter µs | merge µs | step µs | measured MB "
                 "(kernel: bytes, L2 hit) | parity |")
    lines.append("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for r in results:
        us = r.get("us", {})
        res = "; ".join(f"{k}: {v.get('vgprs')} / {v.get('lds')} / {v.get('waves_per_simd')}"
                        for k, v in r.get("resources", {}).items())
        cnt = r.get("counters", {})
        meas = "; ".join(
            f"{k}: {v['bytes'] / 1e6:.1f}, {v['l2_hit']:.2f}" for k, v in sorted(cnt.items())
            if k in ("fwd", "bin_tile", "bin_count", "bin_plan", "bin_scatter", "bin_merge")
            and v.get("bytes") is not None and v.get("l2_hit") is not None)
        par = r.get("parity", {})
        bad = sum(v["outside"] for v in par.values() if isinstance(v, dict))
        par_s = ("ok" if par and bad == 0 else f"{bad} outside") if par else r.get("error", "-")
        lines.append(f"| {r['group']} | {r['name']} ({r.get('schedule', 'auto')}) | "
                     f"{' '.join(r['flags'])} | {r['status']} | "
                     f"{res} | {us.get('fwd', '-')} | {us.get('bin_tile', '-')} | "
                     f"{us.get('bin_count', '-')} | {us.get('bin_plan', '-')} | {us.get('bin_scatter', '-')} | "
                     f"{us.get('bin_merge', '-')} | {us.get('step', '-')} | {meas} | {par_s} |")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    open(path, "w").write("\n".join(lines) + "\n")
    print(f"[sweep] wrote {path}", flush=True)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    b = sub.add_parser("build")
    b.add_argument("--group", action="append", choices=sorted(GROUPS))
    r = sub.add_parser("run")
    r.add_argument("--group", action="append", choices=sorted(GROUPS))
    r.add_argument("--counters", action="store_true")
    r.add_argument("--steps", type=int, default=20)
    r.add_argument("--out", default=os.path.join(ROOT, "profiles", "sweep_encoder.md"))
    o = sub.add_parser("one")
    o.add_argument("--lib", required=True)
    o.add_argument("--workload", type=int, default=2)
    o.add_argument("--steps", type=int, default=20)
    o.add_argument("--ref-dir", required=True)
    o.add_argument("--write-ref", action="store_true")
    o.add_argument("--schedule", default="auto", choices=["auto", "direct", "window"])
    a = ap.parse_args(argv)
    if a.cmd == "build":
        build_points(a.group or sorted(GROUPS))
    elif a.cmd == "run":
        run_points(a.group or sorted(GROUPS), a.counters, a.out, a.steps)
    else:
        print(json.dumps(run_one(a.lib, a.workload, a.steps, a.ref_dir, a.write_ref, a.schedule)),
              flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
