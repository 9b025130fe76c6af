"""Seeded input generators: determinism, shapes, recipes, and the pages' printed shapes."""
import json
import os

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_printed.json")


def test_level_starts_match_printed_examples():
    g = json.load(open(GOLDEN))
    for ex in g["level_starts"]:
        starts = workloads.level_start_index(ex["spatial_shapes"])
        assert starts.tolist() == ex["level_start_index"], ex["cite"]
        assert sum(h * w for h, w in ex["spatial_shapes"]) == ex["S"]


def test_reads_per_query_and_decoder_work():
    g = json.load(open(GOLDEN))
    r = g["reads_per_query"]
    assert r["M"] * r["L"] * r["K"] == r["reads"]
    d = g["decoder_multiply_adds"]
    corner_macs = d["B"] * d["Q"] * d["M"] * d["L"] * d["K"] * 4 * d["D"]
    assert corner_macs == 19_660_800
    assert abs(corner_macs - d["approx"]) <= d["rel_tol"] * d["approx"]


@pytest.mark.parametrize("wid", [0, 1])
def test_deterministic_and_shaped(wid):
    a = workloads.make_inputs(wid)
    b = workloads.make_inputs(wid)
    wl = workloads.WORKLOADS[wid]
    B, Q, M, D, L, K, S = wl.B, wl.num_queries, wl.M, wl.D, wl.L, wl.K, wl.S
    assert a["value"].shape == (B, S, M, D) and a["value"].dtype == np.float32
    assert a["sampling_locations"].shape == (B, Q, M, L, K, 2)
    assert a["attention_weights"].shape == (B, Q, M, L, K)
    assert a["grad_out"].shape == (B, Q, M * D)
    for k in ("value", "sampling_locations", "attention_weights", "grad_out"):
        assert np.array_equal(a[k], b[k])
    np.testing.assert_allclose(a["attention_weights"].sum(axis=(3, 4)), 1.0, rtol=1e-5)


def test_workload_sizes():
    assert workloads.WORKLOADS[2].S == 22223 and workloads.WORKLOADS[2].num_queries == 22223
    assert workloads.WORKLOADS[3].S == 21504
    assert workloads.level_start_index(workloads.PYRAMID_DETR).tolist() == [0, 16700, 20900, 21950]
    assert workloads.level_start_index(workloads.PYRAMID_M2F).tolist() == [0, 16384, 20480]


def test_encoder_references_are_pixel_centres():
    wl = workloads.custom(1, 80, 1, 8, ((8, 8), (4, 4)), 1, ref="pixel_centres", sigma_px=0.0)
    x = workloads.make_inputs(wl, seed=5)
    loc = x["sampling_locations"][0, :, 0, :, 0, :]  # (Q, L, 2)
    # query 9 = level 0, row 1, col 1; query 64 + 5 = level 1, row 1, col 1
    np.testing.assert_allclose(loc[9, 0], [1.5 / 8, 1.5 / 8])
    np.testing.assert_allclose(loc[69, 1], [1.5 / 4, 1.5 / 4])


def test_bf16_rounding_is_exact_and_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], dtype=np.float32)
    r = workloads.round_to_bf16(x)
    bits = r.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    assert r[1] == 1.0 and r[2] == 1.0 + 2 ** -6  # ties to even
    wl = workloads.WORKLOADS[3]
    small = workloads.custom(1, wl.S, 1, 8, wl.shapes, 2, dtype="bf16", ref="pixel_centres")
    arr = workloads.make_inputs(small, seed=3)
    for k in ("value", "sampling_locations", "attention_weights", "grad_out"):
        assert np.all(arr[k].view(np.uint32) & 0xFFFF == 0), k


@pytest.mark.parametrize("kind", ["linear", "morton", "hilbert"])
def test_query_orders_are_level_major_permutations(kind):
    shapes = workloads.PYRAMID_DETR
    order = workloads.query_order(shapes, kind)
    S = sum(h * w for h, w in shapes)
    assert np.array_equal(np.sort(order), np.arange(S))
    base = 0
    for h, w in shapes:  # each level's queries stay in that level's block
        assert set(order[base:base + h * w]) == set(range(base, base + h * w))
        base += h * w


def test_hilbert_order_steps_to_a_neighbour_on_square_levels():
    # on a 2^k x 2^k level the Hilbert curve moves one pixel at a time
    for n in (2, 4, 8, 32):
        r, c = np.divmod(workloads.query_order(((n, n),), "hilbert"), n)
        assert np.all(np.abs(np.diff(r)) + np.abs(np.diff(c)) == 1)
        assert (r[0], c[0]) == (0, 0)


def test_morton_order_is_z_order():
    r, c = np.divmod(workloads.query_order(((4, 4),), "morton"), 4)
    assert list(zip(r[:8], c[:8])) == [(0, 0), (0, 1), (1, 0), (1, 1), (0, 2), (0, 3), (1, 2), (1, 3)]
