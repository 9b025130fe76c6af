"""The binned backward's tile pass has two addressing paths: 32-bit sample-id
division and buffer loads of grad_out rows (taken whenever a launch's ids and
grad_out image stay below 2^31), and 64-bit ids and addresses (taken above
that, at sizes too large to check element by element).  A test hook forces the
64-bit path; both must match the fp64 oracle, and the per-sample gradients of
the two paths must be the same bits (each is computed from the same rows with
the same arithmetic)."""
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
    yield
    msda.msda_test_set_tile_wide_addressing(False)


CASES = {
    "decoder": workloads.WORKLOADS[1],
    "mask2former_bf16": workloads.WORKLOADS[3],
    "ragged_d16": workloads.custom(3, 37, 3, 16, ((7, 9), (4, 5), (1, 3)), 3),
    "d64": workloads.custom(2, 300, 2, 64, ((40, 48), (20, 24)), 4),
}


def _backward(x, wide):
    msda.msda_test_set_tile_wide_addressing(wide)
    try:
        return parity.run_gpu(x)
    finally:
        msda.msda_test_set_tile_wide_addressing(False)


@pytest.mark.parametrize("name", sorted(CASES))
def test_wide_addressing_matches_oracle_and_default(name):
    wl = CASES[name]
    say(f"[tile addressing] {name}: B={wl.B} Q={wl.num_queries} M={wl.M} D={wl.D} "
        f"shapes={wl.shapes} K={wl.K} {wl.dtype}")
    x = workloads.make_inputs(wl, seed=workloads.BASE_SEED + 77)
    want = parity.run_oracle(x)
    wide = _backward(x, True)
    narrow = _backward(x, False)
    tol = TOL_BWD_FP32 if x["dtype"] == "fp32" else HALF_TOL[x["dtype"]]
    for k in ("grad_value", "grad_loc", "grad_attn"):
        check(f"{k} (64-bit path)", wide[k], want[k], *tol)
    assert np.array_equal(wide["grad_loc"], narrow["grad_loc"])
    assert np.array_equal(wide["grad_attn"], narrow["grad_attn"])
