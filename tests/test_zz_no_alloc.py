"""GPU: msda_backward_noalloc (workspace from the library's static per-GPU array)
against msda_backward (workspace from the caller), through the C ABI, on two calls in
a row (the second smaller, so it runs on what the first left in the array), and its
rejection of sizes beyond the array."""
import ctypes

import numpy as np
import pytest
import torch

import parity
import workloads
from parity import HALF_TOL, TOL_BWD_FP32, check, say

import scale_deformable_attention_msda_amd as msda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msda.load_library()


def _both(x, scatter="binned", accum=None):
    t = parity.upload(x)
    ops = parity.operands(t)
    ref = msda.msda_backward(*ops, t["grad_out"], scatter=scatter, accum_dtype=accum,
                             spatial_shapes_host=x["spatial_shapes"])
    gv = torch.full_like(t["value"], float("nan"))
    gl = torch.full_like(t["sampling_locations"], float("nan"))
    ga = torch.full_like(t["attention_weights"], float("nan"))
    got = msda.msda_backward_noalloc(*ops, t["grad_out"], gv, gl, ga, scatter=scatter,
                                     accum_dtype=accum, spatial_shapes_host=x["spatial_shapes"])
    torch.cuda.synchronize()
    return ([r.double().cpu().numpy() for r in ref], [g.double().cpu().numpy() for g in got])


def _compare(x, ref, got):
    tol = TOL_BWD_FP32 if x["dtype"] == "fp32" else HALF_TOL[x["dtype"]]
    for name, r, g in zip(("grad_value", "grad_loc", "grad_attn"), ref, got):
        check(name, g, r, *tol)


def test_noalloc_two_calls_second_smaller():
    free0, _ = torch.cuda.mem_get_info()
    say(f"[noalloc] scratch {msda.msda_noalloc_scratch_bytes()} bytes; encoder workload first")
    x = workloads.make_inputs(2)
    ref, got = _both(x)
    _compare(x, ref, got)
    free1, _ = torch.cuda.mem_get_info()
    say(f"[noalloc] device free memory {free0 / 2**20:.0f} -> {free1 / 2**20:.0f} MiB")
    say("[noalloc] decoder workload second (smaller)")
    x = workloads.make_inputs(1)
    ref, got = _both(x)
    _compare(x, ref, got)
    say("[noalloc] tiny workload third (no scratch needed beyond the counters)")
    x = workloads.make_inputs(0)
    ref, got = _both(x)
    _compare(x, ref, got)


def test_noalloc_atomic_fp32_accumulator_of_bf16():
    wl = workloads.custom(2, 50, 4, 32, ((9, 11), (5, 6)), 4, dtype="bf16")
    x = workloads.make_inputs(wl, seed=5)
    ref, got = _both(x, scatter="atomic")
    _compare(x, ref, got)


def test_noalloc_rejects_sizes_beyond_the_array():
    lib = msda.load_library()
    wl = workloads.WORKLOADS[2]
    dims = msda.MsdaDims(4, wl.S, wl.M, wl.D, wl.L, wl.num_queries, wl.K)  # twice the encoder
    shapes = np.ascontiguousarray(np.array(wl.shapes, dtype=np.int64))
    need = msda.msda_backward_workspace_bytes(dims, msda.MSDA_FP32, msda.MSDA_FP32,
                                              msda.MSDA_SCATTER_BINNED, shapes)
    assert need > msda.msda_noalloc_scratch_bytes()
    st = lib.msda_backward_noalloc(None, None, None, None, None, None, None, None, None,
                                   ctypes.byref(dims), msda.MSDA_FP32, msda.MSDA_FP32,
                                   msda.MSDA_SCATTER_BINNED, shapes.ctypes.data, None)
    assert st == 5  # MSDA_ERR_WORKSPACE
    assert "static scratch" in msda.msda_last_error()
