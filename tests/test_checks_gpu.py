"""GPU tests of the binned backward's device-side checks and of stream handling.

The checks: the kernels compare the device's spatial_shapes / level_start_index
with the plan made from spatial_shapes_host, and the plan pass bounds its waits
on earlier plan blocks.  A failed check writes NaN into every gradient and
leaves a flag that msda_backward_flags reads.  The expired wait is forced from
the host (a zero poll limit), so every kernel still ends normally."""
import numpy as np
import pytest
import torch

import parity
import workloads
from parity import TOL_BWD_FP32, TOL_FWD_FP32, check, say

import scale_deformable_attention_msda_amd as msda

pytestmark = pytest.mark.gpu

DEFAULT_POLLS = 1 << 24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msda.load_library()


def _binned_call(x, t, shapes_host, softmax=False):
    """Backward with an explicit workspace; returns the gradients and the check flags."""
    wl_dims = msda.MsdaDims(*[int(v) for v in (x["value"].shape[0], x["value"].shape[1],
                                                x["value"].shape[2], x["value"].shape[3],
                                                x["spatial_shapes"].shape[0],
                                                x["sampling_locations"].shape[1],
                                                x["sampling_locations"].shape[4])])
    dcode = msda._DTYPES[t["value"].dtype]
    fn = msda.msda_backward_softmax_workspace_bytes if softmax else msda.msda_backward_workspace_bytes
    need = fn(wl_dims, dcode, msda.MSDA_FP32, msda.MSDA_SCATTER_BINNED, shapes_host)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)  # stale contents must not matter
    call = msda.msda_backward_softmax if softmax else msda.msda_backward
    weights = t["attention_logits"] if softmax else t["attention_weights"]
    gv, gl, ga = call(t["value"], t["spatial_shapes"], t["level_start_index"],
                      t["sampling_locations"], weights, t["grad_out"],
                      spatial_shapes_host=shapes_host, workspace=ws)
    flags = msda.msda_backward_flags(wl_dims, dcode, msda.MSDA_FP32, msda.MSDA_SCATTER_BINNED,
                                     softmax, shapes_host, ws)
    torch.cuda.synchronize()
    return gv, gl, ga, flags


def _all_nan(*ts):
    return all(bool(torch.isnan(t).all()) for t in ts)


@pytest.mark.parametrize("softmax", [False, True])
def test_plan_wait_expired_gives_nan_and_flag(softmax):
    # the decoder workload: 6080 bins, 24 plan blocks, so 23 of them wait on predecessors
    x = workloads.make_inputs(1)
    t = parity.upload(x)
    say(f"[checks] plan wait limit 0, decoder workload, softmax={softmax}")
    try:
        msda.msda_test_set_plan_wait_limit(0)
        gv, gl, ga, flags = _binned_call(x, t, x["spatial_shapes"], softmax)
    finally:
        msda.msda_test_set_plan_wait_limit(DEFAULT_POLLS)
    assert flags == msda.MSDA_BWD_PLAN_EXPIRED
    assert _all_nan(gv, gl, ga)
    # the same call with the default limit is valid again (and matches the oracle)
    gv, gl, ga, flags = _binned_call(x, t, x["spatial_shapes"], softmax)
    assert flags == 0
    if not softmax:
        o = parity.run_oracle(x)
        check("grad_value", gv.double().cpu().numpy(), o["grad_value"], *TOL_BWD_FP32)
        check("grad_loc", gl.double().cpu().numpy(), o["grad_loc"], *TOL_BWD_FP32)
        check("grad_attn", ga.double().cpu().numpy(), o["grad_attn"], *TOL_BWD_FP32)


def test_shapes_mismatch_gives_nan_and_flag():
    # device shapes differ from the host copy in one level (same pixel count, so the
    # level starts still agree): the plan and the device disagree
    wl = workloads.custom(2, 40, 4, 32, ((8, 8), (4, 4)), 4)
    x = workloads.make_inputs(wl, seed=11)
    t = parity.upload(x)
    t["spatial_shapes"] = torch.tensor([[8, 8], [2, 8]], dtype=torch.int64, device="cuda")
    say("[checks] device spatial_shapes [[8,8],[2,8]] against host [[8,8],[4,4]]")
    gv, gl, ga, flags = _binned_call(x, t, x["spatial_shapes"])
    assert flags == msda.MSDA_BWD_SHAPES_MISMATCH
    assert _all_nan(gv, gl, ga)


def test_level_start_mismatch_gives_nan_and_flag():
    wl = workloads.custom(2, 40, 4, 32, ((8, 8), (4, 4)), 4)
    x = workloads.make_inputs(wl, seed=12)
    t = parity.upload(x)
    t["level_start_index"] = torch.tensor([0, 63], dtype=torch.int64, device="cuda")
    say("[checks] device level_start_index [0, 63] against the host prefix sums [0, 64]")
    gv, gl, ga, flags = _binned_call(x, t, x["spatial_shapes"])
    assert flags == msda.MSDA_BWD_SHAPES_MISMATCH
    assert _all_nan(gv, gl, ga)


def test_consistent_call_has_no_flags():
    x = workloads.make_inputs(0)
    t = parity.upload(x)
    gv, gl, ga, flags = _binned_call(x, t, x["spatial_shapes"])
    assert flags == 0
    assert not torch.isnan(gv).any() and not torch.isnan(gl).any() and not torch.isnan(ga).any()


@pytest.mark.parametrize("gather,wid", [("direct", 1), ("binned", 2)])
def test_side_stream_not_current(gather, wid):
    """Calls on a stream that is not the current one, with the binding allocating the
    workspaces (they must stay reserved until that stream's work is done).  The binned
    forward needs many queries per region of the finest level: the encoder workload."""
    x = workloads.make_inputs(wid)
    o = parity.run_oracle(x)
    t = parity.upload(x)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    say(f"[checks] workload {wid} on a side stream (not current), gather={gather}")
    outs = []
    for _ in range(3):
        out = msda.msda_forward(*parity.operands(t), stream=s, gather=gather,
                                spatial_shapes_host=x["spatial_shapes"])
        grads = msda.msda_backward(*parity.operands(t), t["grad_out"], stream=s,
                                   spatial_shapes_host=x["spatial_shapes"])
        # allocations on the current stream right away: they must not reuse the workspaces
        junk = [torch.full((1 << 22,), float("nan"), device="cuda") for _ in range(4)]
        outs.append((out, grads, junk))
    s.synchronize()
    torch.cuda.synchronize()
    for out, (gv, gl, ga), _ in outs:
        check("out", out.double().cpu().numpy(), o["out"], *TOL_FWD_FP32)
        check("grad_value", gv.double().cpu().numpy(), o["grad_value"], *TOL_BWD_FP32)
        check("grad_loc", gl.double().cpu().numpy(), o["grad_loc"], *TOL_BWD_FP32)
        check("grad_attn", ga.double().cpu().numpy(), o["grad_attn"], *TOL_BWD_FP32)
