"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle, element by
element, on the same seeded inputs."""
import math
import zlib

import numpy as np
import pytest
import torch

import parity
import workloads
from parity import HALF_TOL, TORCH_DTYPE, TOL_BWD_FP32, TOL_FWD_FP32, check, say

import scale_deformable_attention_msda_amd as msda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msda.load_library()  # raises if the library is not built


def gate(x, g, o, accum_packed=False):
    if x["dtype"] == "fp32":
        check("out", g["out"], o["out"], *TOL_FWD_FP32)
        check("grad_value", g["grad_value"], o["grad_value"], *TOL_BWD_FP32)
        check("grad_loc", g["grad_loc"], o["grad_loc"], *TOL_BWD_FP32)
        check("grad_attn", g["grad_attn"], o["grad_attn"], *TOL_BWD_FP32)
    else:
        tol = HALF_TOL[x["dtype"]]
        check("out", g["out"], o["out"], *tol)
        check("grad_loc", g["grad_loc"], o["grad_loc"], *tol)
        check("grad_attn", g["grad_attn"], o["grad_attn"], *tol)
        if accum_packed:
            say(f"  grad_value (packed {x['dtype']} accumulator, reported): "
                f"{parity.error_stats(g['grad_value'], o['grad_value'])}")
        else:
            check("grad_value", g["grad_value"], o["grad_value"], *tol)


_CACHE = {}


def workload_case(wid):
    """Inputs and oracle results of a workload, computed once per test session."""
    if wid not in _CACHE:
        x = workloads.make_inputs(wid)
        _CACHE.clear()
        _CACHE[wid] = (x, parity.run_oracle(x))
    return _CACHE[wid]


@pytest.mark.parametrize("scatter", ["binned", "atomic"])
@pytest.mark.parametrize("wid", [0, 1, 2, 3, 4])
def test_workload(wid, scatter):
    wl = workloads.WORKLOADS[wid]
    say(f"[parity] workload {wid} {wl.name} B={wl.B} Q={wl.num_queries} M={wl.M} D={wl.D} "
        f"L={wl.L} K={wl.K} {wl.dtype} scatter={scatter}")
    x, o = workload_case(wid)
    g = parity.run_gpu(x, scatter=scatter)
    gate(x, g, o)
    if wl.dtype != "fp32" and scatter == "atomic":
        say(f"  accumulator {wl.dtype}:")
        gate(x, parity.run_gpu(x, accum=TORCH_DTYPE[wl.dtype], scatter="atomic"), o,
             accum_packed=True)


EDGE = {
    # several blocks and a ragged last block (B*Q*M not a multiple of any block size)
    "ragged_fp32": workloads.custom(3, 37, 3, 32, ((7, 9), (4, 5), (1, 3)), 3),
    "ragged_bf16": workloads.custom(3, 37, 3, 32, ((7, 9), (4, 5), (1, 3)), 3, dtype="bf16"),
    "d8_fp32": workloads.custom(2, 50, 4, 8, ((9, 11), (5, 6)), 4),
    "d16_fp32": workloads.custom(2, 50, 4, 16, ((9, 11), (5, 6)), 4),
    "d64_fp32": workloads.custom(2, 50, 4, 64, ((9, 11), (5, 6)), 4),
    "d8_bf16": workloads.custom(2, 50, 4, 8, ((9, 11), (5, 6)), 4, dtype="bf16"),
    "d16_bf16": workloads.custom(2, 50, 4, 16, ((9, 11), (5, 6)), 4, dtype="bf16"),
    "d64_bf16": workloads.custom(2, 50, 4, 64, ((9, 11), (5, 6)), 4, dtype="bf16"),
    "ragged_fp16": workloads.custom(3, 37, 3, 32, ((7, 9), (4, 5), (1, 3)), 3, dtype="fp16"),
    "d8_fp16": workloads.custom(2, 50, 4, 8, ((9, 11), (5, 6)), 4, dtype="fp16"),
    "d16_fp16": workloads.custom(2, 50, 4, 16, ((9, 11), (5, 6)), 4, dtype="fp16"),
    "d64_fp16": workloads.custom(2, 50, 4, 64, ((9, 11), (5, 6)), 4, dtype="fp16"),
    "one_level_one_point": workloads.custom(2, 33, 5, 32, ((6, 10),), 1),
    "max_lk_16_levels": workloads.custom(1, 21, 3, 16, tuple((2 + i % 5, 3 + i % 4) for i in range(16)), 4),
    "max_lk_32_points": workloads.custom(1, 21, 3, 32, ((8, 8), (4, 4)), 32),
    "single_pixel_levels": workloads.custom(2, 19, 2, 32, ((1, 1), (1, 2), (2, 1)), 2, sigma_px=1.0),
    "wide_offsets": workloads.custom(2, 40, 4, 32, ((12, 20), (6, 10)), 4, sigma_px=8.0),
}


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("scatter", ["binned", "atomic"])
def test_edge(name, scatter):
    wl = EDGE[name]
    say(f"[parity] edge {name}: B={wl.B} Q={wl.Q} M={wl.M} D={wl.D} L={wl.L} K={wl.K} {wl.dtype} "
        f"scatter={scatter}")
    x = workloads.make_inputs(wl, seed=zlib.crc32(name.encode()) % 100000)
    o = parity.run_oracle(x)
    gate(x, parity.run_gpu(x, scatter=scatter), o)
    if wl.dtype != "fp32" and scatter == "atomic":
        gate(x, parity.run_gpu(x, accum=TORCH_DTYPE[wl.dtype], scatter="atomic"), o,
             accum_packed=True)


def special_locations():
    """Boundary and non-finite coordinates on power-of-two levels (exact x, y)."""
    wl = workloads.custom(1, 12, 2, 32, ((8, 16), (4, 4)), 4)
    x = workloads.make_inputs(wl, seed=7)
    loc = x["sampling_locations"]
    W0, H0 = 16, 8
    cases = [
        (-0.5 / W0, 0.5),             # x = -1 exactly: forward 0, gradient non-zero
        (-1.5 / W0, 0.5),             # x = -2: wholly outside
        (1.0 + 0.5 / W0, 0.5),        # x = W exactly: wholly outside
        ((W0 - 0.5) / W0, 0.5),       # x = W - 1 exactly (last column centre)
        (0.5, -0.5 / H0),             # y = -1 exactly
        (0.5, 1.0 + 0.5 / H0),        # y = H exactly
        (0.0, 0.0),                   # corner of the map: x = y = -0.5
        (1.0, 1.0),                   # x = W - 0.5, y = H - 0.5
        (math.nan, 0.5), (0.5, math.nan), (math.inf, 0.5), (0.5, -math.inf),
        (1e30, 0.5), (-1e30, -1e30), (3.0, 0.5), (0.5, 3.0),
    ]
    q = 0
    for i, (u, v) in enumerate(cases):
        qq, m, k = (i // 4) % 12, i % 2, i % 4
        loc[0, qq, m, 0, k, 0] = u
        loc[0, qq, m, 0, k, 1] = v
        q = max(q, qq)
    return x


@pytest.mark.parametrize("scatter", ["binned", "atomic"])
def test_boundary_and_nonfinite_locations(scatter):
    say(f"[parity] boundary and non-finite locations, scatter={scatter}")
    x = special_locations()
    o = parity.run_oracle(x)
    g = parity.run_gpu(x, scatter=scatter)
    for k in g:
        assert np.all(np.isfinite(g[k])), k
    gate(x, g, o)


@pytest.mark.parametrize("scatter", ["binned", "atomic"])
def test_empty_queries_zero_grad_value(scatter):
    say(f"[parity] Q = 0: forward is a no-op, backward zero-fills grad_value ({scatter})")
    wl = workloads.custom(2, 0, 2, 32, ((4, 4), (2, 2)), 2)
    x = workloads.make_inputs(wl, seed=1)
    t = parity.upload(x)
    out = msda.msda_forward(*parity.operands(t))
    assert out.shape == (2, 0, 64)
    gv = torch.full_like(t["value"], float("nan"))
    gv, gl, ga = msda.msda_backward(*parity.operands(t), t["grad_out"], grad_value=gv,
                                    scatter=scatter, spatial_shapes_host=x["spatial_shapes"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(gv).item() == 0


def test_batches_split_across_launches():
    """Five 268 MB batch images (48 heads of 64 channels, fp32): more than 2^30 bytes of value,
    so the library runs the batch in two launches (4 + 1 images), for both scatters and the
    softmax method.  Each
    image is checked against the oracle on its own; the pyramid is smaller than num_keys, so
    the rows past it are zeroed in both launches."""
    wl = workloads.custom(5, 40, 48, 64, ((128, 128), (64, 64)), 4)
    extra = 21845 - wl.S
    say(f"[parity] batch over two launches: B=5, S={wl.S}+{extra}, M=48, D=64 (inputs and oracle)")
    x = workloads.make_inputs(wl, seed=41)
    pad = np.random.default_rng(42).standard_normal((wl.B, extra, wl.M, wl.D))
    x["value"] = np.concatenate([x["value"], pad.astype(np.float32)], axis=1)
    assert x["value"].nbytes > 2**30 and 4 * x["value"][0].nbytes < 2**30
    per_image = []
    for b in range(wl.B):
        xb = {k: (v[b:b + 1] if k in parity.FLOAT_KEYS else v) for k, v in x.items()}
        per_image.append((xb, parity.run_oracle(xb)))
    t = parity.upload(x)
    for scatter in ("binned", "atomic"):
        say(f"  scatter={scatter}")
        gv = torch.full_like(t["value"], float("nan"))
        out = msda.msda_forward(*parity.operands(t))
        gv, gl, ga = msda.msda_backward(*parity.operands(t), t["grad_out"], grad_value=gv,
                                        scatter=scatter, spatial_shapes_host=x["spatial_shapes"])
        torch.cuda.synchronize()
        for b, (xb, o) in enumerate(per_image):
            g = {k: v[b:b + 1].double().cpu().numpy() for k, v in
                 dict(out=out, grad_value=gv, grad_loc=gl, grad_attn=ga).items()}
            assert np.all(g["grad_value"][:, -extra:] == 0)
            # grad_value on the (pixel, head) rows either side touches; every other element
            # is zero on both sides, so this is the full element-by-element comparison
            rows = (np.any(o["grad_value"] != 0, axis=(0, 3)) |
                    np.any(g["grad_value"] != 0, axis=(0, 3)))
            g["grad_value"] = g["grad_value"][:, rows]
            gate(xb, g, dict(o, grad_value=o["grad_value"][:, rows]))
        del gv, out, gl, ga
    # the softmax method over the same two launches (binned scatter, L*K = 8: the scatter
    # pass forms the weights itself)
    say("  softmax method")
    ops = (t["value"], t["spatial_shapes"], t["level_start_index"], t["sampling_locations"],
           t["attention_logits"])
    out = msda.msda_forward_softmax(*ops)
    gv, gl, gz = msda.msda_backward_softmax(*ops, t["grad_out"],
                                            spatial_shapes_host=x["spatial_shapes"])
    torch.cuda.synchronize()
    for b, (xb, _) in enumerate(per_image):
        o = parity.run_oracle_softmax(xb)
        g = {k: v[b:b + 1].double().cpu().numpy() for k, v in
             dict(out=out, grad_value=gv, grad_loc=gl, grad_logits=gz).items()}
        rows = (np.any(o["grad_value"] != 0, axis=(0, 3)) |
                np.any(g["grad_value"] != 0, axis=(0, 3)))
        g["grad_value"] = g["grad_value"][:, rows]
        gate_softmax(xb, g, dict(o, grad_value=o["grad_value"][:, rows]))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("scatter", ["binned", "atomic"])
def test_keys_past_the_pyramid(dtype, scatter):
    """num_keys above the pyramid's pixel count (a padded value tensor): the extra key rows are
    never sampled, so every output matches the unpadded call and their gradient rows are zero."""
    wl = workloads.custom(3, 37, 3, 32, ((7, 9), (4, 5), (1, 3)), 3, dtype=dtype)
    extra = 13
    say(f"[parity] {extra} key rows past the pyramid (S = {wl.S} + {extra}), {dtype}, {scatter}")
    x = workloads.make_inputs(wl, seed=31)
    pad = np.random.default_rng(32).standard_normal((wl.B, extra, wl.M, wl.D)).astype(np.float32)
    if dtype == "bf16":
        pad = workloads.round_to_bf16(pad)
    x["value"] = np.concatenate([x["value"], pad], axis=1)
    o = parity.run_oracle(x)
    assert np.all(o["grad_value"][:, -extra:] == 0)
    # garbage in the gradient buffer first: the padded rows must be written, not skipped
    t = parity.upload(x)
    gv = torch.full_like(t["value"], float("nan"))
    out = msda.msda_forward(*parity.operands(t))
    gv, gl, ga = msda.msda_backward(*parity.operands(t), t["grad_out"], grad_value=gv,
                                    scatter=scatter, spatial_shapes_host=x["spatial_shapes"])
    torch.cuda.synchronize()
    g = {k: v.double().cpu().numpy() for k, v in
         dict(out=out, grad_value=gv, grad_loc=gl, grad_attn=ga).items()}
    assert np.all(g["grad_value"][:, -extra:] == 0)
    gate(x, g, o)


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("scatter", ["binned", "atomic"])
def test_outputs_are_overwritten_and_deterministic(dtype, scatter):
    say(f"[parity] overwrite + determinism {dtype} scatter={scatter}")
    wl = workloads.custom(2, 45, 8, 32, workloads.PYRAMID_DETR, 4, dtype=dtype)
    x = workloads.make_inputs(wl, seed=11)
    t = parity.upload(x)
    ops = parity.operands(t)
    junk = lambda like: torch.full_like(like, float("nan"))
    out1 = msda.msda_forward(*ops, out=junk(t["grad_out"]))
    out2 = msda.msda_forward(*ops)
    kw = dict(scatter=scatter, spatial_shapes_host=x["spatial_shapes"])
    gv1, gl1, ga1 = msda.msda_backward(*ops, t["grad_out"], grad_value=junk(t["value"]),
                                       grad_loc=junk(t["sampling_locations"]),
                                       grad_attn=junk(t["attention_weights"]), **kw)
    gv2, gl2, ga2 = msda.msda_backward(*ops, t["grad_out"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2), "forward must be bit-identical across runs"
    assert torch.equal(gl1, gl2) and torch.equal(ga1, ga2)
    for v in (out1, gv1, gl1, ga1):
        assert torch.isfinite(v).all()
    o = parity.run_oracle(x)
    gate(x, {k: v.double().cpu().numpy() for k, v in
             dict(out=out1, grad_value=gv1, grad_loc=gl1, grad_attn=ga1).items()}, o)


def uses_binned_forward(x) -> bool:
    wl = x["workload"]
    d = msda.MsdaDims(wl.B, wl.S, wl.M, wl.D, wl.L, wl.num_queries, wl.K)
    dt = msda._DTYPES[TORCH_DTYPE[x["dtype"]]]
    try:
        return msda.msda_forward_binned_workspace_bytes(d, dt, x["spatial_shapes"]) > 0
    except ValueError:
        return False


def forward_only(x, gather):
    t = parity.upload(x)
    out = msda.msda_forward(*parity.operands(t), gather=gather,
                            spatial_shapes_host=x["spatial_shapes"])
    torch.cuda.synchronize()
    return out


def oracle_forward(x):
    import oracle
    return oracle.forward(x["value"], x["spatial_shapes"], x["level_start_index"],
                          x["sampling_locations"], x["attention_weights"])


def gate_forward(x, out, want):
    tol = TOL_FWD_FP32 if x["dtype"] == "fp32" else HALF_TOL[x["dtype"]]
    check("out", out.double().cpu().numpy(), want, *tol)


@pytest.mark.parametrize("wid", [2, 3, 4])
def test_workload_forward_both_gathers(wid):
    wl = workloads.WORKLOADS[wid]
    say(f"[parity] forward, both gathers: workload {wid} {wl.name}")
    x, o = workload_case(wid)
    assert uses_binned_forward(x), "the query-binned forward should plan this workload"
    for gather in ("binned", "direct"):
        say(f"  gather={gather}")
        gate_forward(x, forward_only(x, gather), o["out"])


# Pyramids with one query per pixel: small enough for the oracle, large enough
# that the query-binned forward plans them (several bins, chunks, windows).
SMALL_PYR = ((20, 30), (10, 15), (5, 8))
SMALL_S = 20 * 30 + 10 * 15 + 5 * 8
SIX_LEVELS = ((24, 32), (12, 16), (6, 8), (3, 4), (2, 2), (1, 1))
BINNED_FWD = {
    "enc_fp32": workloads.custom(2, SMALL_S, 4, 32, SMALL_PYR, 4, ref="pixel_centres"),
    "enc_bf16": workloads.custom(2, SMALL_S, 4, 32, SMALL_PYR, 4, dtype="bf16", ref="pixel_centres"),
    "enc_fp16": workloads.custom(2, SMALL_S, 4, 32, SMALL_PYR, 4, dtype="fp16", ref="pixel_centres"),
    "enc_wide_offsets": workloads.custom(2, SMALL_S, 4, 32, SMALL_PYR, 4, ref="pixel_centres",
                                         sigma_px=7.0),
    "enc_k8": workloads.custom(1, SMALL_S, 4, 32, SMALL_PYR, 8, ref="pixel_centres"),
    "enc_k3": workloads.custom(1, SMALL_S, 3, 32, SMALL_PYR, 3, ref="pixel_centres"),
    "enc_six_levels": workloads.custom(1, 1025, 2, 32, SIX_LEVELS, 4, ref="pixel_centres"),
    "enc_d16_fp32": workloads.custom(2, SMALL_S, 4, 16, SMALL_PYR, 4, ref="pixel_centres"),
    "enc_d64_fp32": workloads.custom(2, SMALL_S, 4, 64, SMALL_PYR, 4, ref="pixel_centres"),
    "enc_d64_bf16": workloads.custom(2, SMALL_S, 4, 64, SMALL_PYR, 4, dtype="bf16",
                                     ref="pixel_centres"),
}


@pytest.mark.parametrize("name", sorted(BINNED_FWD))
def test_binned_forward(name):
    wl = BINNED_FWD[name]
    say(f"[parity] binned forward {name}: B={wl.B} Q={wl.num_queries} M={wl.M} D={wl.D} "
        f"L={wl.L} K={wl.K} {wl.dtype} sigma={wl.sigma_px}")
    x = workloads.make_inputs(wl, seed=zlib.crc32(name.encode()) % 100000, with_grad=False)
    assert uses_binned_forward(x)
    want = oracle_forward(x)
    out1 = forward_only(x, "binned")
    gate_forward(x, out1, want)
    out2 = forward_only(x, "binned")
    assert torch.equal(out1, out2), "forward must be bit-identical across runs"
    gate_forward(x, forward_only(x, "direct"), want)


def test_binned_forward_clustered_and_nonfinite():
    """All points near one spot (bins far above 256 head-queries, cut into chunks),
    plus boundary and non-finite coordinates."""
    say("[parity] binned forward: clustered locations, boundary and non-finite points")
    wl = BINNED_FWD["enc_fp32"]
    x = workloads.make_inputs(wl, seed=5, with_grad=False)
    rng = np.random.default_rng(5)
    loc = x["sampling_locations"]
    loc[...] = (0.5 + 0.01 * rng.standard_normal(loc.shape)).astype(np.float32)
    special = [(math.nan, 0.5), (0.5, math.inf), (-0.5 / 30, 0.5), (1.0, 1.0), (0.0, 0.0),
               (1e30, -1e30), (-math.inf, math.nan)]
    for i, (u, v) in enumerate(special):
        loc[i % 2, 7 * i, i % 4, 0, i % 4, :] = (u, v)
    assert uses_binned_forward(x)
    want = oracle_forward(x)
    out = forward_only(x, "binned")
    assert torch.isfinite(out).all()
    gate_forward(x, out, want)


def test_side_stream():
    say("[parity] non-default stream")
    x = workloads.make_inputs(1)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = parity.run_gpu(x, stream=s)
    gate(x, g, parity.run_oracle(x))


# ---------------------------------------------------------------- softmax method

def gate_softmax(x, g, o):
    fwd, bwd = ((TOL_FWD_FP32, TOL_BWD_FP32) if x["dtype"] == "fp32"
                else (HALF_TOL[x["dtype"]], HALF_TOL[x["dtype"]]))
    check("out", g["out"], o["out"], *fwd)
    for k in ("grad_value", "grad_loc", "grad_logits"):
        check(k, g[k], o[k], *bwd)


@pytest.mark.parametrize("wid,scatter", [(0, "binned"), (0, "atomic"), (1, "binned"),
                                         (1, "atomic"), (2, "binned"), (3, "binned"),
                                         (4, "binned")])
def test_workload_softmax(wid, scatter):
    wl = workloads.WORKLOADS[wid]
    say(f"[parity] softmax method: workload {wid} {wl.name} {wl.dtype} scatter={scatter}")
    x = workloads.make_inputs(wid)
    gate_softmax(x, parity.run_gpu_softmax(x, scatter=scatter), parity.run_oracle_softmax(x))


SOFTMAX_EDGE = ("ragged_fp32", "ragged_bf16", "ragged_fp16", "one_level_one_point",
                "max_lk_16_levels", "max_lk_32_points", "d64_bf16", "d8_fp32")


@pytest.mark.parametrize("name", SOFTMAX_EDGE)
def test_softmax_edge(name):
    wl = EDGE[name]
    say(f"[parity] softmax method, edge {name}: L*K={wl.L * wl.K} D={wl.D} {wl.dtype}")
    x = workloads.make_inputs(wl, seed=zlib.crc32(name.encode()) % 100000)
    o = parity.run_oracle_softmax(x)
    g = parity.run_gpu_softmax(x)
    gate_softmax(x, g, o)
    if wl.L * wl.K == 1:  # one sample per head-query: weight 1, zero logit gradient
        assert np.all(g["grad_logits"] == 0.0)


@pytest.mark.parametrize("name", ["ragged_fp32", "d16_fp32"])
def test_softmax_extreme_logits(name):
    """Shift invariance at large magnitudes, -Inf logits (zero weight), rows of equal
    logits and exp underflow; also that the forward is bit-identical across runs.
    L*K = 9 takes the row pass before the binned scatter, L*K = 8 the weights
    formed inside the scatter pass."""
    say(f"[parity] softmax method: extreme logits, {name}")
    wl = EDGE[name]
    x = workloads.make_inputs(wl, seed=11)
    z = x["attention_logits"]
    B, Q, M = z.shape[:3]
    row = lambda i: (i % B, (3 * i + 1) % Q, i % M)
    z[row(0)] += 3.0e4                        # one row shifted far up
    z[row(1)] -= 3.0e4                        # one far down
    z[row(2)] = 7.25                          # all equal: uniform weights
    z[row(3) + (0, 0)] = -np.inf              # one sample with weight exactly 0
    z[row(4)] = 0.0
    z[row(4) + (0, 0)] = 150.0                # the others underflow in fp32 and fp64 alike
    z[row(5)] *= 60.0                         # a wide spread
    o = parity.run_oracle_softmax(x)
    assert all(np.isfinite(v).all() for v in o.values())
    g = parity.run_gpu_softmax(x)
    gate_softmax(x, g, o)
    t = parity.upload(x)
    ops = (t["value"], t["spatial_shapes"], t["level_start_index"], t["sampling_locations"],
           t["attention_logits"])
    a, b = msda.msda_forward_softmax(*ops), msda.msda_forward_softmax(*ops)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "the softmax forward must be bit-identical across runs"


def test_softmax_matches_plain_method_on_normalised_weights():
    """At full encoder size: the fused softmax forward against msda_forward on weights
    that torch normalised (the two differ only by the fp32 rounding of the weights)."""
    say("[parity] softmax forward vs msda_forward(torch.softmax(logits)), encoder sizes")
    wl = workloads.WORKLOADS[2]
    x = workloads.make_inputs(2, with_grad=False)
    t = parity.upload(x)
    ops = (t["value"], t["spatial_shapes"], t["level_start_index"], t["sampling_locations"])
    z = t["attention_logits"]
    a = torch.softmax(z.reshape(wl.B, -1, wl.M, wl.L * wl.K), dim=-1).reshape(z.shape)
    fused = msda.msda_forward_softmax(*ops, z)
    plain = msda.msda_forward(*ops, a.contiguous())
    torch.cuda.synchronize()
    check("out", fused.double().cpu().numpy(), plain.double().cpu().numpy(), *TOL_FWD_FP32)


# ---------------------------------------------------------- query dispatch order

@pytest.mark.parametrize("kind", ["morton", "hilbert"])
def test_query_order_permutes_outputs(kind):
    """The kernels take head-queries in memory order, so permuting the query axis
    reorders the dispatch.  At encoder size: the forward of the permuted inputs is
    the permutation of the forward, bit for bit (a head-query's sum does not depend
    on its block); the backward's outputs agree within the backward tolerance (the
    order of additions into grad_value, and the fp64 grouping of a sample's
    partial dot products, follow its position in the binned records)."""
    wl = workloads.WORKLOADS[2]
    say(f"[parity] query order {kind}: workload 2 {wl.name}")
    x = workloads.make_inputs(2)
    t = parity.upload(x)
    perm = torch.from_numpy(workloads.query_order(wl.shapes, kind)).cuda()
    pt = dict(t)
    for k in ("sampling_locations", "attention_weights", "grad_out"):
        pt[k] = t[k][:, perm].contiguous()
    host = x["spatial_shapes"]
    out = msda.msda_forward(*parity.operands(t))
    gv, gl, ga = msda.msda_backward(*parity.operands(t), t["grad_out"], spatial_shapes_host=host)
    out_p = msda.msda_forward(*parity.operands(pt))
    gv_p, gl_p, ga_p = msda.msda_backward(*parity.operands(pt), pt["grad_out"],
                                          spatial_shapes_host=host)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out[:, perm]), "forward must not depend on the dispatch order"
    np_ = lambda v: v.double().cpu().numpy()
    check("grad_value", np_(gv_p), np_(gv), *TOL_BWD_FP32)
    check("grad_loc", np_(gl_p), np_(gl[:, perm]), *TOL_BWD_FP32)
    check("grad_attn", np_(ga_p), np_(ga[:, perm]), *TOL_BWD_FP32)


# ---------------------------------------------------------------- fp16 at full size

# Workload 5: the Mask2Former configuration of workload 3 (B=2, Q=S=21504, M=8,
# D=32, three levels 128x128 / 64x64 / 32x32, K=4, pixel-centre references) in
# IEEE fp16.
M2F_FP16 = workloads.WORKLOADS[5]


@pytest.mark.parametrize("scatter", ["binned", "atomic"])
def test_fp16_mask2former_size(scatter):
    say(f"[parity] fp16, Mask2Former sizes, scatter={scatter}")
    x = workloads.make_inputs(5)
    o = parity.run_oracle(x)
    gate(x, parity.run_gpu(x, scatter=scatter), o)
    gate_forward(x, forward_only(x, "binned"), o["out"])
    if scatter == "atomic":
        say("  accumulator fp16:")
        gate(x, parity.run_gpu(x, accum=torch.float16, scatter="atomic"), o, accum_packed=True)


def test_fp16_softmax_mask2former_size():
    say("[parity] fp16 softmax method, Mask2Former sizes")
    x = workloads.make_inputs(5)
    gate_softmax(x, parity.run_gpu_softmax(x), parity.run_oracle_softmax(x))


# ---------------------------------------------------------------- HIP graphs

@pytest.mark.parametrize("scatter", ["binned", "atomic"])
def test_graph_capture_replays_match_eager(scatter):
    """Forward + backward captured once in a HIP graph (torch.cuda.CUDAGraph) and
    replayed several times, with eager work and synchronisations between the
    replays: every replay matches the eager call (forward, grad_loc and grad_attn
    bit for bit; grad_value within the backward tolerance, since its additions
    are unordered) and the oracle.  Fill kernels, not memsets, clear the
    accumulators and counters, so nothing in the graph is a memset node."""
    wl = workloads.WORKLOADS[1]
    say(f"[parity] graph capture: workload 1 {wl.name} scatter={scatter}")
    x, o = workload_case(1)
    t = parity.upload(x)
    ops = parity.operands(t)
    host = x["spatial_shapes"]
    out_e = msda.msda_forward(*ops)
    gv_e, gl_e, ga_e = msda.msda_backward(*ops, t["grad_out"], scatter=scatter,
                                          spatial_shapes_host=host)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the allocator outside the capture
        msda.msda_backward(*ops, t["grad_out"], scatter=scatter, spatial_shapes_host=host)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_g = msda.msda_forward(*ops)
        gv_g, gl_g, ga_g = msda.msda_backward(*ops, t["grad_out"], scatter=scatter,
                                              spatial_shapes_host=host)
    for rep in range(3):
        for v in (out_g, gv_g, gl_g, ga_g):
            v.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}: forward differs from eager"
        assert torch.equal(gl_g, gl_e) and torch.equal(ga_g, ga_e), f"replay {rep}"
        np_ = lambda v: v.double().cpu().numpy()
        check(f"replay {rep} grad_value vs eager", np_(gv_g), np_(gv_e), *TOL_BWD_FP32)
    gate(x, {k: v.double().cpu().numpy() for k, v in
             dict(out=out_g, grad_value=gv_g, grad_loc=gl_g, grad_attn=ga_g).items()}, o)


# ------------------------------------------------- binned forward, order reused

def test_binned_forward_reuse_order():
    """msda_forward_binned_reuse walks the query order an earlier call left in the
    workspace: on the same inputs it repeats that call bit for bit, and on other
    inputs of the same sizes (other offsets, so other regions) it is still exact."""
    wl = BINNED_FWD["enc_fp32"]
    say("[parity] binned forward, order reused across inputs")
    xa = workloads.make_inputs(wl, seed=101, with_grad=False)
    xb = workloads.make_inputs(wl, seed=202, with_grad=False)
    ta, tb = parity.upload(xa), parity.upload(xb)
    d = msda.MsdaDims(wl.B, wl.S, wl.M, wl.D, wl.L, wl.num_queries, wl.K)
    host = xa["spatial_shapes"]
    ws = torch.empty(msda.msda_forward_binned_workspace_bytes(d, msda.MSDA_FP32, host),
                     dtype=torch.uint8, device="cuda")
    kw = dict(gather="binned", spatial_shapes_host=host, workspace=ws)
    out_a = msda.msda_forward(*parity.operands(ta), **kw)
    out_b = msda.msda_forward(*parity.operands(tb), reuse_order=True, **kw)
    out_a2 = msda.msda_forward(*parity.operands(ta), reuse_order=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_a2, out_a), "same order and inputs must repeat bit for bit"
    gate_forward(xb, out_b, oracle_forward(xb))


def test_binned_forward_reuse_order_encoder_size():
    say("[parity] binned forward, order of other inputs reused, encoder sizes")
    wl = workloads.WORKLOADS[2]
    x, o = workload_case(2)
    other = workloads.make_inputs(2, seed=workloads.BASE_SEED + 77, with_grad=False)
    d = msda.MsdaDims(wl.B, wl.S, wl.M, wl.D, wl.L, wl.num_queries, wl.K)
    host = x["spatial_shapes"]
    ws = torch.empty(msda.msda_forward_binned_workspace_bytes(d, msda.MSDA_FP32, host),
                     dtype=torch.uint8, device="cuda")
    kw = dict(gather="binned", spatial_shapes_host=host, workspace=ws)
    msda.msda_forward(*parity.operands(parity.upload(other)), **kw)
    out = msda.msda_forward(*parity.operands(parity.upload(x)), reuse_order=True, **kw)
    torch.cuda.synchronize()
    gate_forward(x, out, o["out"])
