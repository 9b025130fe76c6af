"""Build ``libmsda.so`` (the C-ABI MSDA library) for gfx950 with hipcc, in-tree.

Each source compiles to an object of its own (in parallel), then hipcc links
the shared library.  ``extra_flags`` (e.g. ``-DMSDA_BIN_TILE=10``) reach every
compile, which is how the tuning sweep builds its variants.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libmsda.so")
SOURCES = ["msda_api.hip", "msda_kernels.hip", "msda_binned.hip", "msda_fwd_binned.hip",
           "msda_profile.hip", "msda_microbench.hip", "msda_noalloc.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the device code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
_NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd: list[str], remarks: list[str] | None = None) -> None:
    proc = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in proc.stderr.splitlines() if _NOISE not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{' '.join(cmd)}\n{err}")
    if remarks is not None:
        remarks.append(err)
    elif err.strip():
        print(err, file=sys.stderr)


def build(out: str = LIB_PATH, extra_flags: list[str] | None = None, jobs: int | None = None,
          remarks: list[str] | None = None) -> str:
    """Compile and link the library into `out`; with `remarks`, the compilers' diagnostics
    are appended there instead of printed."""
    tmpdir = tempfile.mkdtemp(prefix="msda_build_")
    try:
        objs, cmds = [], []
        for s in SOURCES:
            obj = os.path.join(tmpdir, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            cmds.append([hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC,
                         "-c", "-o", obj, os.path.join(CSRC, s)])
        workers = jobs or min(len(cmds), os.cpu_count() or 1, 8)
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, c, remarks) for c in cmds]:
                f.result()
        tmp = out + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(extra_flags=sys.argv[1:]))
