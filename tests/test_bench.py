"""bench.py end to end: on the GPU one short run prints one JSON line with the
fields the benchmark contract names, a roofline object for the dominant
kernel and a CPU baseline of the oracle; --gpus above 1 is refused."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=240):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=timeout, cwd=ROOT)


@pytest.mark.gpu
def test_bench_json_line():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = run_bench("--steps", "3", "--warmup", "1", "--no-extras", "--workload", "1")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is False and d["value"] > 0
    assert d["config"]["workload"].startswith("decoder")
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert 0 < rl["frac"] < 1 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1


def test_bench_refuses_more_than_one_gpu():  # exits before touching torch: runs on the CPU
    r = run_bench("--gpus", "2", timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
