"""GPU parity of the forward's two schedules against the fp64 oracle.

The LDS-window schedule keeps the small levels of one (batch, head) whole in LDS
and a window of rows of the next level, and gathers everything else (and every
sample whose cell leaves the window) from global memory.  The launch picks it on
its own for large query counts (the encoder workloads of test_parity_gpu run
it); here a test hook forces it on small inputs, whose pyramids put levels
whole in LDS, in a window with fallbacks, or not at all, and on boundary and
non-finite locations, for both the plain and the softmax method."""
import zlib

import numpy as np
import pytest
import torch

import parity
import workloads
from parity import HALF_TOL, TOL_FWD_FP32, check, say

import scale_deformable_attention_msda_amd as msda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msda.load_library()
    yield
    msda.msda_test_set_forward_schedule("auto")


CASES = {
    # every level whole in LDS
    "small_fp32": workloads.custom(2, 300, 4, 32, ((9, 11), (5, 6)), 4),
    # level 1 whole (32 KB), level 0 in a window of a few rows with most samples falling back
    "window_fp32": workloads.custom(1, 700, 2, 32, ((64, 64), (16, 16)), 4),
    # the same with the reference points at pixel centres (raster order), as in the encoder
    "window_pixel_refs": workloads.custom(1, 4352, 2, 32, ((64, 64), (16, 16)), 4,
                                          ref="pixel_centres"),
    "window_d64": workloads.custom(1, 500, 2, 64, ((48, 40), (12, 10), (6, 5)), 4),
    "window_d8": workloads.custom(2, 400, 3, 8, ((200, 180), (50, 45)), 3),
    "window_bf16": workloads.custom(1, 700, 2, 32, ((96, 96), (24, 24)), 4, dtype="bf16"),
    "window_fp16": workloads.custom(1, 700, 2, 32, ((96, 96), (24, 24)), 4, dtype="fp16"),
    # no level fits with enough rows: everything from global memory
    "all_global": workloads.custom(1, 200, 2, 64, ((400, 300),), 2),
    "ragged": workloads.custom(3, 37, 3, 32, ((7, 9), (4, 5), (1, 3)), 3),
    "lk9_wide": workloads.custom(2, 333, 2, 32, ((40, 70), (20, 35), (10, 17)), 3, sigma_px=8.0),
    "single_pixel_levels": workloads.custom(2, 19, 2, 32, ((1, 1), (1, 2), (2, 1)), 2),
}


def _tol(dtype):
    return TOL_FWD_FP32 if dtype == "fp32" else HALF_TOL[dtype]


def _forward(x, schedule, softmax=False):
    t = parity.upload(x)
    msda.msda_test_set_forward_schedule(schedule)
    try:
        if softmax:
            out = msda.msda_forward_softmax(*parity.operands(t)[:4], t["attention_logits"])
        else:
            out = msda.msda_forward(*parity.operands(t))
        torch.cuda.synchronize()
    finally:
        msda.msda_test_set_forward_schedule("auto")
    return out.double().cpu().numpy()


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("softmax", [False, True])
def test_window_schedule_matches_oracle(name, softmax):
    wl = CASES[name]
    say(f"[window] {name}: B={wl.B} Q={wl.Q} M={wl.M} D={wl.D} shapes={wl.shapes} K={wl.K} "
        f"{wl.dtype} softmax={softmax}")
    x = workloads.make_inputs(wl, seed=zlib.crc32(name.encode()) % 100000)
    if softmax:
        import oracle
        want = oracle.forward_softmax(x["value"], x["spatial_shapes"], x["level_start_index"],
                                      x["sampling_locations"], x["attention_logits"])
    else:
        want = parity.run_oracle(x)["out"]
    got_w = _forward(x, "window", softmax)
    got_d = _forward(x, "direct", softmax)
    check("out (window)", got_w, want, *_tol(x["dtype"]))
    check("out (direct)", got_d, want, *_tol(x["dtype"]))


def test_window_schedule_boundary_and_nonfinite():
    from test_parity_gpu import special_locations

    x = special_locations()
    want = parity.run_oracle(x)["out"]
    got = _forward(x, "window")
    assert np.all(np.isfinite(got))
    check("out (window)", got, want, *TOL_FWD_FP32)


def test_window_schedule_is_deterministic():
    x = workloads.make_inputs(CASES["window_pixel_refs"], seed=3)
    a = _forward(x, "window")
    b = _forward(x, "window")
    assert np.array_equal(a, b)
