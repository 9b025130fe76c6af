"""The grid_sample composition that the layer-level comparison measures
against (bench.grid_sample_msda_softmax), checked on the CPU in fp64 against
the oracle's softmax-method forward, so that the comparison computes the same
operator."""
import numpy as np
import pytest
import torch

import bench
import oracle
import workloads


@pytest.mark.parametrize("name,wl", [
    ("tiny", workloads.WORKLOADS[0]),
    ("ragged", workloads.custom(2, 37, 3, 16, ((7, 9), (4, 5), (1, 3)), 3)),
    ("wide", workloads.custom(1, 40, 2, 8, ((12, 20), (6, 10)), 4, sigma_px=8.0)),
])
def test_grid_sample_composition_matches_oracle(name, wl):
    x = workloads.make_inputs(wl, seed=31, with_grad=False)
    args = [x[k] for k in ("value", "spatial_shapes", "level_start_index", "sampling_locations")]
    want = oracle.forward_softmax(*args, x["attention_logits"])
    t = lambda k: torch.from_numpy(np.ascontiguousarray(x[k])).double()
    got = bench.grid_sample_msda_softmax(t("value"), None, None, t("sampling_locations"),
                                         t("attention_logits"), x["spatial_shapes"])
    np.testing.assert_allclose(got.numpy().reshape(want.shape), want, rtol=1e-12, atol=1e-12)
