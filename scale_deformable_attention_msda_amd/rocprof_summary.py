"""Summaries of rocprofv3 output for profiles/ (kernel traces, traffic, counters).

  python -m scale_deformable_attention_msda_amd.rocprof_summary trace DIR --title T --command C
      per-kernel calls / average / min / max / share from DIR's *kernel_stats.csv
  python -m scale_deformable_attention_msda_amd.rocprof_summary traffic --fetch DIR --write DIR
         --copy-fetch DIR --copy-write DIR --workload encoder --scatter binned --command C
      bytes per launch of every library kernel: FETCH_SIZE and WRITE_SIZE (KiB per dispatch,
      the runs' means) each scaled by what the same counter reads for a plain copy of known
      size, plus the L2 hit rate when the write run also holds TCC_HIT_sum / TCC_MISS_sum.
      bench.py reads the 'traffic' and 'l2hit' lines while the kernel sources hash to the
      digest written beside them.
  python -m scale_deformable_attention_msda_amd.rocprof_summary counters DIR [DIR ...] --command C
      per-kernel means of every counter in the directories (one pass each), with derived
      ratios (time waiting, VALU issue, L1 / L2 hit rates, L2 latency, LDS bank conflicts)
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 256 * 2 ** 20  # the plain copy `bench.py --calibrate-copy` makes

# library profile names (bench.py's) of the kernels, by function name
PROFILE_NAME = {"fwd_kernel": "fwd", "fwd_win_kernel": "fwd", "tile_kernel": "bin_tile",
                "count_kernel": "bin_count", "scatter_kernel": "bin_scatter",
                "merge_kernel": "bin_merge", "plan_kernel": "bin_plan", "zero_kernel": "zero",
                "bwd_kernel": "bwd_atomic", "cast_kernel": "cast",
                "softmax_rows_kernel": "softmax_rows",
                "softmax_grad_rows_kernel": "softmax_grad_rows"}


def kernel_base(name: str) -> str:
    """'void msda::(anonymous namespace)::tile_kernel<float, 32>(msda::BinArgs)' -> 'tile_kernel'."""
    base = name.replace("(anonymous namespace)", "").split("<")[0].split("(")[0]
    return base.split("::")[-1].strip()


def pretty(name: str) -> str:
    return name.replace("void ", "").replace("msda::(anonymous namespace)::", "").split("(msda::")[0]


def counter_means(d: str) -> dict:
    """{kernel full name: {counter: mean value per dispatch}} over d's counter files."""
    acc = collections.defaultdict(lambda: collections.defaultdict(dict))
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                per = acc[row["Kernel_Name"]][row["Counter_Name"]]
                did = row["Dispatch_Id"]
                per[did] = per.get(did, 0.0) + float(row["Counter_Value"] or 0)
    return {k: {c: sum(v.values()) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def trace(d: str, title: str, command: str) -> str:
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(files[0], newline="")))
    lines = [f"# Kernel trace: {title}", "", "Command (repository root on the GPU host, "
             "`cd /tmp && export TMPDIR=/tmp` first):", "", f"    {command}", "",
             "Durations in microseconds (rocprofv3 --kernel-trace --stats).", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {pretty(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    return "\n".join(lines) + "\n"


def traffic(fetch: str, write: str, copy_fetch: str, copy_write: str, workload: str,
            scatter: str, command: str) -> str:
    sys.path.insert(0, ROOT)
    import bench  # the digest of the kernel sources

    cf = [v for k, v in counter_means(copy_fetch).items() if "copy" in k.lower()]
    cw = [v for k, v in counter_means(copy_write).items() if "copy" in k.lower()]
    if not cf or not cw:
        raise SystemExit("no copy kernel in the calibration runs")
    f_scale = COPY_BYTES / (cf[0]["FETCH_SIZE"] * 1024)
    w_scale = COPY_BYTES / (cw[0]["WRITE_SIZE"] * 1024)
    fm, wm = counter_means(fetch), counter_means(write)
    lines = [f"# HBM traffic per launch, {workload} workload, scatter {scatter}, from rocprofv3 counters",
             "#", "# Commands (GPU host, cd /tmp && export TMPDIR=/tmp):", f"#   {command}",
             "#", f"# Calibration: the 256 MiB copy reads FETCH_SIZE {cf[0]['FETCH_SIZE']:.0f} KiB and "
             f"WRITE_SIZE {cw[0]['WRITE_SIZE']:.0f} KiB per launch,",
             f"# so FETCH_SIZE is scaled by {f_scale:.3f} and WRITE_SIZE by {w_scale:.3f} to bytes.",
             "# Rows: kernel, FETCH_SIZE KiB, WRITE_SIZE KiB (means over the run's launches), traffic "
             "bytes = scaled sum; l2hit = TCC_HIT / (TCC_HIT + TCC_MISS).",
             "# bench.py reads the 'traffic' and 'l2hit' lines; they apply only while the kernel "
             "sources hash to 'sources'.", f"sources: {bench.kernel_source_digest()}"]
    for name in sorted(set(fm) & set(wm)):
        key = PROFILE_NAME.get(kernel_base(name))
        if key is None:
            continue
        fk, wk = fm[name].get("FETCH_SIZE"), wm[name].get("WRITE_SIZE")
        if fk is None or wk is None:
            continue
        lines.append(f"# {pretty(name)}: FETCH_SIZE {fk:.1f} KiB, WRITE_SIZE {wk:.1f} KiB")
        lines.append(f"traffic {workload}/{scatter}/{key}: {fk * 1024 * f_scale + wk * 1024 * w_scale:.0f}")
        hit, miss = wm[name].get("TCC_HIT_sum"), wm[name].get("TCC_MISS_sum")
        if hit is not None and miss is not None and hit + miss > 0:
            lines.append(f"l2hit {workload}/{scatter}/{key}: {hit / (hit + miss):.4f}")
    return "\n".join(lines) + "\n"


def _ratio(cs: dict, num: str, den: str, one_minus: bool = False):
    if num not in cs or not cs.get(den):
        return None
    r = cs[num] / cs[den]
    return 1.0 - r if one_minus else r


def counters(dirs: list[str], command: str, title: str = "") -> str:
    merged = collections.defaultdict(dict)
    for d in dirs:
        for k, cs in counter_means(d).items():
            merged[k].update(cs)
    names = sorted((k for k in merged if kernel_base(k) in PROFILE_NAME), key=kernel_base)
    lines = ["# Hardware counters per launch (means over each run's dispatches)", "",
             *([title, ""] if title else []),
             "Commands (GPU host, `cd /tmp && export TMPDIR=/tmp`; one pass per counter group):", "",
             f"    {command}", "",
             "SQ_* counters are summed over the device, TCC_* over the L2 channels of the 8 XCDs, "
             "TCP_* over the vector L1s.", "",
             "Columns: waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES; issuing VALU = SQ_ACTIVE_INST_VALU / "
             "SQ_WAVE_CYCLES; L1 hit = 1 - TCP_TCC_READ_REQ / TCP_TOTAL_CACHE_ACCESSES; L2 hit = "
             "TCC_HIT / (TCC_HIT + TCC_MISS); L2 latency = TCP_TCC_READ_REQ_LATENCY / "
             "TCP_TCC_READ_REQ (cycles, seen from the L1); LDS conflict = SQ_LDS_BANK_CONFLICT / "
             "SQ_ACTIVE_INST_LDS.", "",
             "| kernel | waves | VALU insts | LDS insts | VMEM rd / wr insts | waiting | issuing VALU "
             "| L1 hit | L2 hit | L2 latency | LDS conflict |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]

    def f(x, fmt):
        return "-" if x is None else format(x, fmt)

    for k in names:
        cs = merged[k]
        l2 = None
        if "TCC_HIT_sum" in cs and cs.get("TCC_HIT_sum", 0) + cs.get("TCC_MISS_sum", 0) > 0:
            l2 = cs["TCC_HIT_sum"] / (cs["TCC_HIT_sum"] + cs["TCC_MISS_sum"])
        m = lambda c: None if c not in cs else cs[c] / 1e6
        lines.append(
            f"| {pretty(k)} | {f(cs.get('SQ_WAVES'), ',.0f')} | {f(m('SQ_INSTS_VALU'), '.2f')} M | "
            f"{f(m('SQ_INSTS_LDS'), '.2f')} M | {f(m('SQ_INSTS_VMEM_RD'), '.2f')} / "
            f"{f(m('SQ_INSTS_VMEM_WR'), '.2f')} M | "
            f"{f(_ratio(cs, 'SQ_WAIT_ANY', 'SQ_WAVE_CYCLES'), '.2f')} | "
            f"{f(_ratio(cs, 'SQ_ACTIVE_INST_VALU', 'SQ_WAVE_CYCLES'), '.2f')} | "
            f"{f(_ratio(cs, 'TCP_TCC_READ_REQ_sum', 'TCP_TOTAL_CACHE_ACCESSES_sum', True), '.2f')} | "
            f"{f(l2, '.2f')} | "
            f"{f(_ratio(cs, 'TCP_TCC_READ_REQ_LATENCY_sum', 'TCP_TCC_READ_REQ_sum'), '.0f')} | "
            f"{f(_ratio(cs, 'SQ_LDS_BANK_CONFLICT', 'SQ_ACTIVE_INST_LDS'), '.2f')} |")
    lines += ["", "Raw means per launch:", ""]
    for k in names:
        lines.append(f"- {pretty(k)}: " + ", ".join(f"{c} {v:.4g}" for c, v in sorted(merged[k].items())))
    return "\n".join(lines) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    f = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy-fetch", "copy-write", "workload", "scatter", "command"):
        f.add_argument("--" + k, required=True)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--command", required=True)
    c.add_argument("--title", default="")
    for p in (t, f, c):
        p.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        text = trace(a.dir, a.title, a.command)
    elif a.cmd == "traffic":
        text = traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.workload, a.scatter, a.command)
    else:
        text = counters(a.dirs, a.command, a.title)
    open(a.out, "w").write(text)
    print(f"wrote {a.out}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
