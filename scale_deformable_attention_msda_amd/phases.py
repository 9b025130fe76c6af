"""Where the binned backward's tile pass spends its time, phase by phase.

A diagnostic build of the library (-DMSDA_TILE_PHASE_CLOCKS) has every wave
of a tile block read the shader clock after each phase of a chunk.  The
library keeps wave 0's sums per block.  This module builds that library
beside the in-tree one, runs the binned backward on the encoder workload, and
writes each phase's share of the blocks' clocks, and that share of the tile
pass's HIP-event duration, to a profiles/ summary.

  python -m scale_deformable_attention_msda_amd.phases build       (any host: compile)
  python -m scale_deformable_attention_msda_amd.phases run [--launches N]
         [--out profiles/tile_phases_encoder.md]                    (GPU)

Wave 0 also plans each chunk's items, so its view shows the block's critical
path through the planning phase.  Two tile blocks share a CU, so a phase's
wall time is not all lost issue time: the other block's waves run meanwhile.
The clock reads cost a few instructions per phase (the diagnostic build's tile
pass is a little slower than the default one).
"""
from __future__ import annotations

import argparse
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(ROOT, "_build", "phases", "libmsda.so")
PHASES = ["staging and chunk claim", "cell pass", "cell scan, plan and record sort", "item loop",
          "next chunk's position", "next chunk's loads issued", "result pass", "pixel pass",
          "last barrier"]


def build() -> str:
    from scale_deformable_attention_msda_amd import build as b
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    return b.build(out=LIB, extra_flags=["-DMSDA_TILE_PHASE_CLOCKS"])


def run(launches: int, out: str) -> None:
    import torch
    sys.path.insert(0, ROOT)
    import workloads
    import scale_deformable_attention_msda_amd as msda

    msda.load_library(LIB)
    wl = workloads.WORKLOADS[2]
    x = workloads.make_inputs(wl)
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(x[k]).to(dev) for k in
         ("value", "sampling_locations", "attention_weights", "grad_out", "spatial_shapes",
          "level_start_index")}
    ops = (t["value"], t["spatial_shapes"], t["level_start_index"], t["sampling_locations"],
           t["attention_weights"])
    host = x["spatial_shapes"]
    for _ in range(3):
        msda.msda_backward(*ops, t["grad_out"], spatial_shapes_host=host)
    torch.cuda.synchronize()
    sums = [0.0] * 12
    tile_us = []
    blocks = 0
    for _ in range(launches):
        msda.msda_profile_select("bin_tile")
        msda.msda_profile_start(64)
        msda.msda_backward(*ops, t["grad_out"], spatial_shapes_host=host)
        torch.cuda.synchronize()
        tile_us += [ms * 1e3 for name, ms in msda.msda_profile_stop(64) if name == "bin_tile"]
        rows = [r for r in msda.msda_test_tile_phase_clocks() if r[11] > 0]
        blocks = len(rows)
        for r in rows:
            for k in range(12):
                sums[k] += r[k]
    msda.msda_profile_select(None)
    total = sum(sums[:len(PHASES)])
    chunks = sums[11]
    us = sum(tile_us) / len(tile_us)
    lines = ["# Tile pass phases: encoder workload, binned backward", "",
             "Workload: B=2, Q=S=22223, M=8, D=32, L=4 (100x167, 50x84, 25x42, 13x21), K=4, fp32; "
             "one MI355X.", "",
             "Command (repository root on the GPU host; the diagnostic library is built beforehand on "
             "any host with `python -m scale_deformable_attention_msda_amd.phases build`):", "",
             f"    python -m scale_deformable_attention_msda_amd.phases run --launches {launches}", "",
             "Each tile block's wave 0 reads the shader clock (s_memtime) after every phase of a "
             "chunk; the shares are of the summed clocks over all blocks and launches. `us` = share x "
             "the diagnostic build's mean tile-pass HIP-event duration. Two blocks share each CU, so "
             "a phase's wall time overlaps the other block's work.", "",
             f"Launches: {launches}; tile blocks: {blocks}; chunks per launch: {chunks / launches:.0f}; "
             f"tile pass (diagnostic build): {us:.1f} us per launch.", "",
             "| phase | share | us | clocks per chunk |", "|---|---|---|---|"]
    for k, name in enumerate(PHASES):
        share = sums[k] / total if total else 0.0
        lines.append(f"| {name} | {share * 100:.1f}% | {share * us:.1f} | "
                     f"{sums[k] / chunks if chunks else 0:.0f} |")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("build")
    r = sub.add_parser("run")
    r.add_argument("--launches", type=int, default=5)
    r.add_argument("--out", default=os.path.join(ROOT, "profiles", "tile_phases_encoder.md"))
    a = ap.parse_args(argv)
    if a.cmd == "build":
        print(build())
    else:
        run(a.launches, a.out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
