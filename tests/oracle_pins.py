"""Pins of the fp64 oracle against things other than itself.

Each ``pin_*`` function takes an oracle object (``forward``/``backward``
methods, see ``oracle.Oracle``) and raises AssertionError when the oracle
disagrees with what the pages or the mathematics fix.  The tests run every pin
against the real oracle, and run them against deliberately broken copies of
the oracle to show that each plausible mistake is caught by at least one pin.

Independent formulations used here (none of them calls the oracle's code):
  * a brute-force forward that evaluates every bilinear sample as an explicit
    sum over all pixels of the level with tent weights
    tri(x - j) * tri(y - i), tri(t) = max(0, 1 - |t|).  For a finite point
    this equals the four-corner rule with zero padding of chapter 1 of the
    msda-triton course ("Bilinear interpolation: reading between the
    pixels"), since only the (at most) four pixels within distance 1 in both
    axes get a non-zero tent weight, and they get exactly the corner weights;
  * torch.nn.functional.grid_sample(align_corners=False, padding_mode="zeros")
    in fp64 on the CPU, which the same section names as the equivalent
    library routine, with grid = 2 * loc - 1;
  * closed forms: a constant field, an affine field, pixel-centre points
    that reduce the operator to a plain gather (forward) and a plain
    scatter-add (grad_value);
  * finite differences, which are exact up to rounding here: the output is
    linear in the attention weights and in the value, and linear in x for a
    fixed y inside one cell;
  * the adjoint identity <F(V), G> = <V, F^T(G)> for the linear map V -> out;
  * for the "softmax" method: torch.softmax and its autograd in fp64, the
    invariants sum A = 1 and sum grad_logits = 0, and central differences of
    the whole operator with a numpy softmax.
"""
from __future__ import annotations

import numpy as np

import workloads


# ----------------------------------------------------------------- problems

def random_problem(seed, B=2, Q=5, M=3, D=4, shapes=((5, 7), (3, 4), (2, 2)), K=3,
                   lo=-0.3, hi=1.3):
    """A tiny random problem whose points may leave [0, 1] (partially or wholly)."""
    rng = np.random.default_rng(seed)
    L = len(shapes)
    S = sum(h * w for h, w in shapes)
    return dict(
        value=rng.standard_normal((B, S, M, D)),
        spatial_shapes=np.asarray(shapes, dtype=np.int64),
        level_start_index=workloads.level_start_index(shapes),
        sampling_locations=rng.uniform(lo, hi, (B, Q, M, L, K, 2)),
        attention_weights=rng.random((B, Q, M, L, K)),
        grad_out=rng.standard_normal((B, Q, M * D)),
    )


def operands(p):
    return (p["value"], p["spatial_shapes"], p["level_start_index"], p["sampling_locations"],
            p["attention_weights"])


def interior_locations(rng, shape, shapes):
    """Points whose four corners all lie inside their level: x in [0, W-1)."""
    B, Q, M, L, K = shape
    loc = np.empty((B, Q, M, L, K, 2))
    for l, (h, w) in enumerate(shapes):
        x = rng.uniform(0.0, w - 1.0, (B, Q, M, K))
        y = rng.uniform(0.0, h - 1.0, (B, Q, M, K))
        loc[:, :, :, l, :, 0] = (x + 0.5) / w
        loc[:, :, :, l, :, 1] = (y + 0.5) / h
    return loc


# -------------------------------------------------------------- brute force

def tent_forward(value, spatial_shapes, level_start_index, sampling_locations,
                 attention_weights):
    """Forward as an explicit tent-weighted sum over every pixel of every level."""
    value = np.asarray(value, dtype=np.float64)
    B, S, M, D = value.shape
    Q = sampling_locations.shape[1]
    out = np.zeros((B, Q, M, D))
    for l, (h, w) in enumerate(np.asarray(spatial_shapes)):
        s0 = int(level_start_index[l])
        V = value[:, s0:s0 + h * w].reshape(B, h, w, M, D)
        x = sampling_locations[:, :, :, l, :, 0] * w - 0.5
        y = sampling_locations[:, :, :, l, :, 1] * h - 0.5
        tx = np.maximum(0.0, 1.0 - np.abs(x[..., None] - np.arange(w)))
        ty = np.maximum(0.0, 1.0 - np.abs(y[..., None] - np.arange(h)))
        a = attention_weights[:, :, :, l, :]
        out += np.einsum("bqmk,bqmki,bqmkj,bijmd->bqmd", a, ty, tx, V)
    return out.reshape(B, Q, M * D)


def grid_sample_forward(value, spatial_shapes, level_start_index, sampling_locations,
                        attention_weights, requires_grad=False):
    """Forward via torch grid_sample per level (fp64, CPU), summed over levels."""
    import torch
    import torch.nn.functional as F

    v = torch.tensor(np.asarray(value, dtype=np.float64), requires_grad=requires_grad)
    loc = torch.tensor(np.asarray(sampling_locations, dtype=np.float64),
                       requires_grad=requires_grad)
    a = torch.tensor(np.asarray(attention_weights, dtype=np.float64),
                     requires_grad=requires_grad)
    B, S, M, D = v.shape
    Q, K = loc.shape[1], loc.shape[4]
    out = torch.zeros(B, M, D, Q, dtype=torch.float64)
    for l, (h, w) in enumerate(np.asarray(spatial_shapes)):
        s0 = int(level_start_index[l])
        img = v[:, s0:s0 + h * w].reshape(B, h, w, M, D).permute(0, 3, 4, 1, 2)
        img = img.reshape(B * M, D, h, w)
        grid = (2.0 * loc[:, :, :, l] - 1.0).permute(0, 2, 1, 3, 4).reshape(B * M, Q, K, 2)
        samp = F.grid_sample(img, grid, mode="bilinear", padding_mode="zeros",
                             align_corners=False)  # (B*M, D, Q, K)
        wl = a[:, :, :, l].permute(0, 2, 1, 3).reshape(B * M, 1, Q, K)
        out = out + (samp * wl).sum(-1).reshape(B, M, D, Q)
    out = out.permute(0, 3, 1, 2).reshape(B, Q, M * D)
    return out, (v, loc, a)


# ---------------------------------------------------------------------- pins

def _close(got, want, atol, what):
    err = np.max(np.abs(np.asarray(got) - np.asarray(want))) if np.size(want) else 0.0
    assert err <= atol, f"{what}: max |err| = {err:.3e} > {atol:.1e}"


def pin_forward_tent_sum(orc):
    for seed in range(4):
        p = random_problem(seed)
        _close(orc.forward(*operands(p)), tent_forward(*operands(p)), 1e-12,
               f"forward vs tent sum (seed {seed})")
    # a single-level pyramid with one column / one row, and many points far outside
    p = random_problem(7, shapes=((1, 6), (4, 1)), lo=-1.5, hi=2.5)
    _close(orc.forward(*operands(p)), tent_forward(*operands(p)), 1e-12,
           "forward vs tent sum (degenerate levels)")


def pin_forward_grid_sample(orc):
    for seed in (11, 12):
        p = random_problem(seed)
        ref, _ = grid_sample_forward(*operands(p))
        _close(orc.forward(*operands(p)), ref.detach().numpy(), 1e-12,
               f"forward vs grid_sample (seed {seed})")


def pin_constant_field(orc):
    """Bilinear weights sum to 1: a constant field returns gamma * sum(a)."""
    rng = np.random.default_rng(21)
    shapes = ((6, 9), (3, 5))
    B, Q, M, D, K = 2, 4, 2, 3, 3
    S = sum(h * w for h, w in shapes)
    gamma = np.array([1.0, -2.5, 0.125])
    value = np.broadcast_to(gamma, (B, S, M, D)).copy()
    loc = interior_locations(rng, (B, Q, M, len(shapes), K), shapes)
    a = rng.random((B, Q, M, len(shapes), K))
    out = orc.forward(value, np.asarray(shapes), workloads.level_start_index(shapes), loc, a)
    want = a.sum(axis=(3, 4))[..., None] * gamma
    _close(out.reshape(B, Q, M, D), want, 1e-13, "constant field")


def _affine_problem(seed):
    rng = np.random.default_rng(seed)
    shapes = ((6, 9), (4, 3))
    B, Q, M, D, K = 1, 3, 2, 2, 2
    L = len(shapes)
    starts = workloads.level_start_index(shapes)
    S = sum(h * w for h, w in shapes)
    alpha, beta, gamma = rng.standard_normal((3, M, D))
    value = np.empty((B, S, M, D))
    for l, (h, w) in enumerate(shapes):
        i, j = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
        field = (alpha[None, None] * j[..., None, None] + beta[None, None] * i[..., None, None]
                 + gamma[None, None])
        value[:, starts[l]:starts[l] + h * w] = field.reshape(h * w, M, D)[None]
    loc = interior_locations(rng, (B, Q, M, L, K), shapes)
    a = rng.random((B, Q, M, L, K))
    g = rng.standard_normal((B, Q, M * D))
    return shapes, starts, value, loc, a, g, (alpha, beta, gamma)


def pin_affine_field(orc):
    """Bilinear interpolation reproduces an affine field exactly inside the map, and the
    location gradient of <out, g> is (a W <g, alpha>, a H <g, beta>)."""
    shapes, starts, value, loc, a, g, (alpha, beta, gamma) = _affine_problem(31)
    B, Q, M, L, K = a.shape
    D = value.shape[-1]
    want = np.zeros((B, Q, M, D))
    gl_want = np.zeros(loc.shape)
    for l, (h, w) in enumerate(shapes):
        x = loc[:, :, :, l, :, 0] * w - 0.5
        y = loc[:, :, :, l, :, 1] * h - 0.5
        al = a[:, :, :, l, :]
        want += np.einsum("bqmk,md->bqmd", al * x, alpha)
        want += np.einsum("bqmk,md->bqmd", al * y, beta)
        want += np.einsum("bqmk,md->bqmd", al, gamma)
        gq = g.reshape(B, Q, M, D)
        gl_want[:, :, :, l, :, 0] = al * w * np.einsum("bqmd,md->bqm", gq, alpha)[..., None]
        gl_want[:, :, :, l, :, 1] = al * h * np.einsum("bqmd,md->bqm", gq, beta)[..., None]
    ops = (value, np.asarray(shapes), starts, loc, a)
    _close(orc.forward(*ops).reshape(B, Q, M, D), want, 1e-12, "affine field forward")
    _, gl, _ = orc.backward(*ops, g)
    _close(gl, gl_want, 1e-11, "affine field grad_loc")


def _pixel_centre_problem(seed):
    """Power-of-two levels and points on pixel centres: x = j, y = i exactly."""
    rng = np.random.default_rng(seed)
    shapes = ((8, 16), (4, 4), (2, 8))
    B, Q, M, D, K = 2, 5, 3, 4, 3
    L = len(shapes)
    starts = workloads.level_start_index(shapes)
    S = sum(h * w for h, w in shapes)
    value = rng.standard_normal((B, S, M, D))
    rows = np.empty((B, Q, M, L, K), dtype=np.int64)
    loc = np.empty((B, Q, M, L, K, 2))
    for l, (h, w) in enumerate(shapes):
        i = rng.integers(0, h, (B, Q, M, K))
        j = rng.integers(0, w, (B, Q, M, K))
        loc[:, :, :, l, :, 0] = (j + 0.5) / w
        loc[:, :, :, l, :, 1] = (i + 0.5) / h
        rows[:, :, :, l, :] = starts[l] + i * w + j
    a = rng.random((B, Q, M, L, K))
    g = rng.standard_normal((B, Q, M * D))
    return shapes, starts, value, loc, a, g, rows


def pin_pixel_centres_gather_scatter(orc):
    shapes, starts, value, loc, a, g, rows = _pixel_centre_problem(41)
    B, Q, M, L, K = a.shape
    D = value.shape[-1]
    ops = (value, np.asarray(shapes), starts, loc, a)
    # forward = plain gather of the addressed rows, weighted by a
    want = np.zeros((B, Q, M, D))
    for b in range(B):
        for m in range(M):
            picked = np.take(value[b, :, m, :], rows[b, :, m].reshape(-1), axis=0)
            want[b, :, m] = np.einsum("qn,qnd->qd", a[b, :, m].reshape(Q, -1),
                                      picked.reshape(Q, L * K, D))
    _close(orc.forward(*ops).reshape(B, Q, M, D), want, 1e-13, "pixel centres forward")
    # grad_value = plain scatter-add of a * g onto the addressed rows
    gv_want = np.zeros_like(value)
    gq = g.reshape(B, Q, M, D)
    for b in range(B):
        for m in range(M):
            idx = rows[b, :, m].reshape(-1)
            contrib = (a[b, :, m].reshape(Q, L * K)[..., None] * gq[b, :, m][:, None, :])
            np.add.at(gv_want[b, :, m, :], idx, contrib.reshape(-1, D))
    gv, _, ga = orc.backward(*ops, g)
    _close(gv, gv_want, 1e-13, "pixel centres grad_value")
    # grad_attn = <g, addressed value row>
    ga_want = np.zeros((B, Q, M, L * K))
    for b in range(B):
        for m in range(M):
            picked = np.take(value[b, :, m, :], rows[b, :, m].reshape(-1), axis=0)
            ga_want[b, :, m] = np.einsum("qd,qnd->qn", gq[b, :, m], picked.reshape(Q, L * K, D))
    _close(ga.reshape(B, Q, M, L * K), ga_want, 1e-13, "pixel centres grad_attn")


def _loss(orc_or_fn, ops, g):
    out = orc_or_fn(*ops)
    return float(np.sum(out * g))


def pin_grad_attn(orc):
    """Output is linear in a: central differences are exact up to rounding, and
    sum_{l,k} a * grad_attn = <out, g> per (b, q, m)."""
    p = random_problem(51, B=1, Q=3, M=2, D=3, shapes=((4, 5), (2, 3)), K=2)
    ops = list(operands(p))
    g = p["grad_out"]
    _, _, ga = orc.backward(*ops, g)
    a = ops[4]
    fd = np.empty_like(a)
    h = 1e-3
    for idx in np.ndindex(a.shape):
        ap, am = a.copy(), a.copy()
        ap[idx] += h
        am[idx] -= h
        fd[idx] = (_loss(tent_forward, ops[:4] + [ap], g)
                   - _loss(tent_forward, ops[:4] + [am], g)) / (2 * h)
    _close(ga, fd, 1e-9, "grad_attn vs central differences")
    B, Q, M = a.shape[:3]
    out = orc.forward(*ops).reshape(B, Q, M, -1)
    lhs = np.sum(a * ga, axis=(3, 4))
    rhs = np.einsum("bqmd,bqmd->bqm", out, g.reshape(B, Q, M, -1))
    _close(lhs, rhs, 1e-12, "sum a*grad_attn = <out, g>")


def pin_grad_value_adjoint(orc):
    """<F(V), G> = <V, F^T(G)> for random V, G (the forward is linear in V)."""
    for seed in (61, 62):
        p = random_problem(seed)
        ops = operands(p)
        gv, _, _ = orc.backward(*ops, p["grad_out"])
        lhs = float(np.sum(tent_forward(*ops) * p["grad_out"]))
        rhs = float(np.sum(p["value"] * gv))
        assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs)), \
            f"adjoint identity: {lhs!r} vs {rhs!r}"
        # the scatter touches each value element through F's rows only: a second,
        # independent random V must satisfy the identity too
        v2 = np.random.default_rng(seed + 100).standard_normal(p["value"].shape)
        lhs2 = float(np.sum(tent_forward(v2, *ops[1:]) * p["grad_out"]))
        rhs2 = float(np.sum(v2 * gv))
        assert abs(lhs2 - rhs2) <= 1e-11 * max(1.0, abs(lhs2)), "adjoint identity (2nd V)"


def _far_from_edges(x, margin):
    return np.abs(x - np.round(x)) > margin


def pin_grad_loc_central_differences(orc):
    """grad_loc against central differences of the tent-sum forward, for points whose
    pixel coordinates are at least 1e-4 px from any integer (no kink inside +-h)."""
    p = random_problem(71, B=1, Q=3, M=2, D=3, shapes=((4, 5), (3, 2)), K=2, lo=-0.25, hi=1.25)
    ops = list(operands(p))
    g = p["grad_out"]
    _, gl, _ = orc.backward(*ops, g)
    loc = ops[3]
    h = 1e-7
    checked = 0
    for idx in np.ndindex(loc.shape):
        l, axis = idx[3], idx[5]
        H, W = p["spatial_shapes"][l]
        size = W if axis == 0 else H
        coord = loc[idx] * size - 0.5
        if not _far_from_edges(coord, 1e-4):
            continue
        lp, lm = loc.copy(), loc.copy()
        lp[idx] += h
        lm[idx] -= h
        fd = (_loss(tent_forward, ops[:3] + [lp, ops[4]], g)
              - _loss(tent_forward, ops[:3] + [lm, ops[4]], g)) / (2 * h)
        assert abs(gl[idx] - fd) <= 1e-6 * max(1.0, abs(fd)), \
            f"grad_loc{idx}: {gl[idx]!r} vs central difference {fd!r}"
        checked += 1
    assert checked > 0.9 * loc.size


def pin_grad_loc_right_derivative_on_edges(orc):
    """On a cell edge (pixel centre, and x = -1 where the forward contribution is 0 but the
    gradient is not) the oracle's grad_loc is the derivative from the right, the side that
    floor assigns the point to."""
    shapes = ((4, 8), (2, 4))
    rng = np.random.default_rng(81)
    B, Q, M, D, K = 1, 2, 1, 3, 2
    L = len(shapes)
    starts = workloads.level_start_index(shapes)
    S = sum(h * w for h, w in shapes)
    value = rng.standard_normal((B, S, M, D))
    loc = np.empty((B, Q, M, L, K, 2))
    for l, (h, w) in enumerate(shapes):
        j = rng.integers(-1, w, (B, Q, M, K))   # includes x = -1 exactly
        i = rng.integers(0, h, (B, Q, M, K))
        loc[:, :, :, l, :, 0] = (j + 0.5) / w
        loc[:, :, :, l, :, 1] = (i + 0.5) / h
    loc[0, 0, 0, 0, 0, 0] = -0.5 / shapes[0][1]  # x = -1 exactly
    a = rng.random((B, Q, M, L, K)) + 0.5
    g = rng.standard_normal((B, Q, M * D))
    ops = [value, np.asarray(shapes), starts, loc, a]
    _, gl, _ = orc.backward(*ops, g)
    h = 2.0 ** -20
    base = _loss(tent_forward, ops, g)
    for idx in np.ndindex(loc.shape):
        lp = loc.copy()
        lp[idx] += h
        fd = (_loss(tent_forward, ops[:3] + [lp, a], g) - base) / h
        assert abs(gl[idx] - fd) <= 1e-6 * max(1.0, abs(fd)), \
            f"right derivative {idx}: {gl[idx]!r} vs {fd!r}"
    assert abs(gl[0, 0, 0, 0, 0, 0]) > 1e-3, "x = -1 must carry a non-zero gradient"


def pin_autograd_grid_sample(orc):
    """All three gradients against torch autograd through fp64 grid_sample, for points
    off cell edges (grid_sample's own edge convention is not assumed)."""
    import torch

    p = random_problem(91, B=2, Q=4, M=2, D=3, shapes=((5, 6), (3, 3)), K=2)
    ops = operands(p)
    for l, (h, w) in enumerate(p["spatial_shapes"]):
        for axis, size in ((0, w), (1, h)):
            c = p["sampling_locations"][:, :, :, l, :, axis] * size - 0.5
            near = ~_far_from_edges(c, 1e-6)
            p["sampling_locations"][:, :, :, l, :, axis][near] += 3e-6 / size
    out, (v, loc, a) = grid_sample_forward(*ops, requires_grad=True)
    (out * torch.tensor(p["grad_out"])).sum().backward()
    gv, gl, ga = orc.backward(*ops, p["grad_out"])
    _close(gv, v.grad.numpy(), 1e-12, "grad_value vs autograd")
    _close(gl, loc.grad.numpy(), 1e-10, "grad_loc vs autograd")
    _close(ga, a.grad.numpy(), 1e-12, "grad_attn vs autograd")


def pin_out_of_range_and_nonfinite(orc):
    """Wholly-outside points contribute nothing and get zero gradients; NaN and infinite
    coordinates are treated as outside; partially-outside points follow the tent sum."""
    p = random_problem(101, B=1, Q=4, M=2, D=3, shapes=((4, 4), (2, 3)), K=3)
    loc = p["sampling_locations"]
    w0 = p["spatial_shapes"][0][1]
    loc[0, 0, :, 0, 0, 0] = -1.5 / w0 - 0.01     # x < -1: wholly left
    loc[0, 0, :, 0, 1, 0] = 1.0 + 0.6 / w0        # x >= W: wholly right
    loc[0, 1, :, 1, 0, 1] = np.nan
    loc[0, 1, :, 1, 1, 0] = np.inf
    loc[0, 1, :, 1, 2, 1] = -np.inf
    loc[0, 2, :, 0, 2, :] = 1e30
    loc[0, 3, :, 0, 0, 0] = -0.4 / w0             # partially outside (x in (-1, 0))
    ops = operands(p)
    out = orc.forward(*ops)
    assert np.all(np.isfinite(out))
    dead = np.zeros(p["attention_weights"].shape, dtype=bool)
    dead[0, 0, :, 0, 0] = dead[0, 0, :, 0, 1] = True
    dead[0, 1, :, 1, :] = True
    dead[0, 2, :, 0, 2] = True
    # the forward equals the tent sum over the remaining (finite) points only
    a_live = np.where(dead, 0.0, p["attention_weights"])
    loc_finite = np.where(np.isfinite(loc), loc, 0.0)
    _close(out, tent_forward(p["value"], p["spatial_shapes"], p["level_start_index"],
                             loc_finite, a_live), 1e-12, "forward with dead points")
    gv, gl, ga = orc.backward(*ops, p["grad_out"])
    assert np.all(ga[dead] == 0.0) and np.all(gl[dead] == 0.0)
    assert np.all(np.isfinite(gv)) and np.all(np.isfinite(gl)) and np.all(np.isfinite(ga))


def _softmax_np(z):
    """Softmax over the last two axes (L, K) of z, written out in numpy for the pins."""
    sh = z.shape
    z2 = z.reshape(sh[:3] + (-1,))
    e = np.exp(z2 - z2.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).reshape(sh)


def pin_softmax_library(orc):
    """The "softmax" method against torch.softmax in fp64, its derivative against
    torch autograd, the weights summing to 1, grad_logits summing to 0 per
    head-query, and constant logits giving exactly 1 / (L K)."""
    import torch

    rng = np.random.default_rng(71)
    z = rng.standard_normal((2, 3, 2, 3, 4)) * 3.0
    a = orc.softmax(z)
    zt = torch.tensor(z.reshape(2, 3, 2, 12), dtype=torch.float64, requires_grad=True)
    at = torch.softmax(zt, dim=-1)
    _close(a.reshape(2, 3, 2, 12), at.detach().numpy(), 1e-15, "softmax vs torch.softmax")
    ga = rng.standard_normal(a.shape)
    (at * torch.tensor(ga.reshape(2, 3, 2, 12))).sum().backward()
    gz = orc.softmax_backward(a, ga)
    _close(gz.reshape(2, 3, 2, 12), zt.grad.numpy(), 1e-14, "softmax derivative vs autograd")
    _close(a.sum(axis=(3, 4)), np.ones((2, 3, 2)), 1e-15, "weights sum to 1")
    _close(gz.sum(axis=(3, 4)), np.zeros((2, 3, 2)), 1e-13, "grad_logits sum to 0")
    c = orc.softmax(np.full((1, 2, 1, 2, 3), 5.0))
    assert np.all(c == 1.0 / 6.0), "constant logits give uniform weights"


def pin_softmax_composition(orc):
    """grad_logits of the operator with softmax weights against central
    differences of the tent-sum forward with a numpy softmax."""
    p = random_problem(81, B=1, Q=2, M=2, D=3, shapes=((4, 5), (2, 3)), K=2)
    ops = list(operands(p))[:4]
    g = p["grad_out"]
    z = np.random.default_rng(82).standard_normal(p["attention_weights"].shape)
    out = orc.forward_softmax(*ops, z)
    _close(out, tent_forward(*ops, _softmax_np(z)), 1e-12, "forward with softmax weights")
    _, _, gz = orc.backward_softmax(*ops, z, g)
    fd = np.empty_like(z)
    h = 1e-5
    for idx in np.ndindex(z.shape):
        zp, zm = z.copy(), z.copy()
        zp[idx] += h
        zm[idx] -= h
        fd[idx] = (_loss(tent_forward, ops + [_softmax_np(zp)], g)
                   - _loss(tent_forward, ops + [_softmax_np(zm)], g)) / (2 * h)
    _close(gz, fd, 1e-8, "grad_logits vs central differences")


ALL_PINS = [
    pin_forward_tent_sum,
    pin_forward_grid_sample,
    pin_constant_field,
    pin_affine_field,
    pin_pixel_centres_gather_scatter,
    pin_grad_attn,
    pin_grad_value_adjoint,
    pin_grad_loc_central_differences,
    pin_grad_loc_right_derivative_on_edges,
    pin_autograd_grid_sample,
    pin_out_of_range_and_nonfinite,
    pin_softmax_library,
    pin_softmax_composition,
]
