"""Seeded synthetic inputs for the MSDA operator.

This module builds inputs only.  It holds none of the operator's arithmetic
(no sampling, no interpolation, no gradients), and both the GPU path's tests
and the fp64 oracle consume exactly the arrays it returns.

Workloads (shapes as the pages describe the operator's tensors, chapter 1 of
the msda-triton course, "The equation, term by term"):

  id  name         B  Q         M  D   levels (H x W)                     K  dtype  offsets
  0   tiny         1  16        2  8   8x8, 4x4                           2  fp32   N(0, 1.5 px)
  1   decoder      2  300       8  32  100x167, 50x84, 25x42, 13x21       4  fp32   N(0, 2 px)
  2   encoder      2  S=22223   8  32  100x167, 50x84, 25x42, 13x21       4  fp32   N(0, 2 px)
  3   mask2former  2  S=21504   8  32  128x128, 64x64, 32x32              4  bf16   N(0, 2 px)
  4   contention   1  S=22223   8  32  100x167, 50x84, 25x42, 13x21       8  bf16   N(0, 0.5 px)
  5   m2f_fp16     2  S=21504   8  32  128x128, 64x64, 32x32              4  fp16   N(0, 2 px)

Workload 5 is workload 3 in IEEE binary16, the other half-precision type the
DeformOps page names (introduction: bfloat16 and float16 throughout).

The 4-level pyramid is that of an ~800x1333 detection input at strides 8, 16,
32 and 64 (chapter 1, "The problem: attention over images is quadratic"); the
3-level one stands in for the Mask2Former pixel-decoder encoder (DeformOps
page, introduction: 5k to 22k queries per call).  They are synthetic stand-ins
for those workloads: no image, dataset or trained weight is involved.

Recipe (numpy ``Generator(PCG64(seed))``, default seed 20261202 + id), drawn in
this order:
  1. value ~ N(0, 1), shape (B, S, M, D);
  2. reference points: workloads 0-1 draw one point ~ U[0, 1]^2 per (b, q);
     workloads 2-4 put query i on the centre of the i-th pixel of the
     flattened pyramid (level-major, row-major), ((c + 0.5)/W, (r + 0.5)/H) of
     its own level, shared by all levels;
  3. offsets ~ N(0, sigma px) per (b, q, m, l, k, axis), divided by W_l for x
     and by H_l for y, added to the reference point;
  4. logits ~ N(0, 1), shape (B, Q, M, L*K); weights = fp64 softmax over the
     L*K axis, then rounded to the workload's dtype; the logits themselves
     (less their per-row maximum) are kept as attention_logits for the
     "softmax" method;
  5. grad_out ~ N(0, 1), shape (B, Q, M*D).
For bf16 (fp16) workloads every floating array is rounded to bf16 (IEEE
binary16), round to nearest even, and returned as float32 holding exactly
representable values, so that both the GPU path (which converts exactly) and
the oracle (which upcasts exactly to
fp64) see identical numbers.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PYRAMID_DETR = ((100, 167), (50, 84), (25, 42), (13, 21))
PYRAMID_M2F = ((128, 128), (64, 64), (32, 32))
BASE_SEED = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    M: int
    D: int
    shapes: tuple
    K: int
    dtype: str          # "fp32", "bf16" or "fp16"
    ref: str            # "uniform" or "pixel_centres"
    sigma_px: float
    Q: int | None = None  # None: one query per pyramid pixel (Q = S)
    extra: dict = field(default_factory=dict)

    @property
    def L(self) -> int:
        return len(self.shapes)

    @property
    def S(self) -> int:
        return int(sum(h * w for h, w in self.shapes))

    @property
    def num_queries(self) -> int:
        return self.S if self.Q is None else self.Q


WORKLOADS = {
    0: Workload("tiny", B=1, Q=16, M=2, D=8, shapes=((8, 8), (4, 4)), K=2, dtype="fp32",
                ref="uniform", sigma_px=1.5),
    1: Workload("decoder", B=2, Q=300, M=8, D=32, shapes=PYRAMID_DETR, K=4, dtype="fp32",
                ref="uniform", sigma_px=2.0),
    2: Workload("encoder", B=2, M=8, D=32, shapes=PYRAMID_DETR, K=4, dtype="fp32",
                ref="pixel_centres", sigma_px=2.0),
    3: Workload("mask2former", B=2, M=8, D=32, shapes=PYRAMID_M2F, K=4, dtype="bf16",
                ref="pixel_centres", sigma_px=2.0),
    4: Workload("contention", B=1, M=8, D=32, shapes=PYRAMID_DETR, K=8, dtype="bf16",
                ref="pixel_centres", sigma_px=0.5),
    5: Workload("m2f_fp16", B=2, M=8, D=32, shapes=PYRAMID_M2F, K=4, dtype="fp16",
                ref="pixel_centres", sigma_px=2.0),
}


def level_start_index(shapes) -> np.ndarray:
    """Exclusive prefix sum of H*W over the levels (DeformOps page, layer example)."""
    sizes = [int(h) * int(w) for h, w in shapes]
    return np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    # finite values never carry out of the top bit here; NaNs are restored below
    rounded = (bits + (np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))))
    rounded &= np.uint32(0xFFFF0000)
    out = rounded.view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out


def pixel_centre_refs(shapes) -> np.ndarray:
    """(x, y) of every pyramid pixel centre, normalised per level; shape (S, 2)."""
    refs = []
    for h, w in shapes:
        r, c = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
        refs.append(np.stack([(c.ravel() + 0.5) / w, (r.ravel() + 0.5) / h], axis=-1))
    return np.concatenate(refs, axis=0)  # (S, 2), level-major, row-major


def _morton_key(r: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Z-order key: the bits of row and column interleaved (column in the even bits)."""
    key = np.zeros(r.shape, dtype=np.int64)
    for bit in range(16):
        key |= ((c >> bit) & 1) << (2 * bit)
        key |= ((r >> bit) & 1) << (2 * bit + 1)
    return key


def _hilbert_key(r: np.ndarray, c: np.ndarray, n: int) -> np.ndarray:
    """Distance along the Hilbert curve over an n x n grid (n a power of two) of
    cell (x = c, y = r): at each scale s the quadrant adds s^2 * (3 rx xor ry),
    and the coordinates are reflected and swapped into that quadrant's frame."""
    x, y = c.astype(np.int64).copy(), r.astype(np.int64).copy()
    d = np.zeros(x.shape, dtype=np.int64)
    s = n // 2
    while s > 0:
        rx = ((x & s) > 0).astype(np.int64)
        ry = ((y & s) > 0).astype(np.int64)
        d += s * s * ((3 * rx) ^ ry)
        flip = (ry == 0) & (rx == 1)
        x = np.where(flip, s - 1 - x, x)
        y = np.where(flip, s - 1 - y, y)
        swap = ry == 0
        x, y = np.where(swap, y, x), np.where(swap, x, y)
        x &= s - 1
        y &= s - 1
        s //= 2
    return d


def query_order(shapes, kind: str) -> np.ndarray:
    """A dispatch order of the encoder's queries (one per pyramid pixel, level-major,
    row-major): position i of the result is the query visited i-th.  "linear"
    keeps raster order; "morton" and "hilbert" visit each level's pixels along
    that space-filling curve, levels still in order."""
    if kind not in ("linear", "morton", "hilbert"):
        raise ValueError(f"unknown query order {kind!r}")
    order, base = [], 0
    for h, w in shapes:
        r, c = np.divmod(np.arange(h * w, dtype=np.int64), w)
        if kind == "linear":
            key = np.arange(h * w)
        elif kind == "morton":
            key = _morton_key(r, c)
        else:
            n = 1 << int(np.ceil(np.log2(max(h, w, 1))))
            key = _hilbert_key(r, c, n)
        order.append(base + np.argsort(key, kind="stable"))
        base += h * w
    return np.concatenate(order)


def make_inputs(wl: Workload | int, seed: int | None = None, with_grad: bool = True) -> dict:
    """Build one workload's operands as numpy arrays (see the module docstring)."""
    if isinstance(wl, int):
        if seed is None:
            seed = BASE_SEED + wl
        wl = WORKLOADS[wl]
    if seed is None:
        seed = BASE_SEED
    rng = np.random.Generator(np.random.PCG64(seed))
    B, M, D, K, L, S, Q = wl.B, wl.M, wl.D, wl.K, wl.L, wl.S, wl.num_queries
    shapes = np.asarray(wl.shapes, dtype=np.int64).reshape(L, 2)

    value = rng.standard_normal((B, S, M, D), dtype=np.float32)
    if wl.ref == "uniform":
        ref = rng.random((B, Q, 2))
        ref = ref[:, :, None, None, None, :]
    elif wl.ref == "pixel_centres":
        if Q != S:
            raise ValueError("pixel-centre references need one query per pyramid pixel")
        ref = pixel_centre_refs(wl.shapes)[None, :, None, None, None, :]
    else:
        raise ValueError(f"unknown reference-point recipe {wl.ref!r}")
    offsets = rng.standard_normal((B, Q, M, L, K, 2)) * wl.sigma_px
    scale = np.stack([shapes[:, 1], shapes[:, 0]], axis=-1).astype(np.float64)  # (W_l, H_l)
    loc = ref + offsets / scale[None, None, None, :, None, :]
    logits = rng.standard_normal((B, Q, M, L * K))
    logits -= logits.max(axis=-1, keepdims=True)
    e = np.exp(logits)
    weights = (e / e.sum(axis=-1, keepdims=True)).reshape(B, Q, M, L, K)
    grad_out = rng.standard_normal((B, Q, M * D), dtype=np.float32) if with_grad else None

    arrays = {
        "value": value,
        "sampling_locations": loc.astype(np.float32),
        "attention_weights": weights.astype(np.float32),
        # the same logits, raw, for the "softmax" method (weights normalised
        # inside the operator); drawn above, so nothing else changes
        "attention_logits": logits.reshape(B, Q, M, L, K).astype(np.float32),
    }
    if grad_out is not None:
        arrays["grad_out"] = grad_out
    if wl.dtype == "bf16":
        arrays = {k: round_to_bf16(v) for k, v in arrays.items()}
    elif wl.dtype == "fp16":
        # numpy's float32 -> float16 conversion rounds to nearest even
        arrays = {k: v.astype(np.float16).astype(np.float32) for k, v in arrays.items()}
    elif wl.dtype != "fp32":
        raise ValueError(f"unsupported dtype {wl.dtype!r}")
    arrays["spatial_shapes"] = shapes
    arrays["level_start_index"] = level_start_index(wl.shapes)
    arrays["dtype"] = wl.dtype
    arrays["workload"] = wl
    return arrays


def custom(B, Q, M, D, shapes, K, dtype="fp32", ref="uniform", sigma_px=2.0) -> Workload:
    """A workload of arbitrary shape, for edge-case tests."""
    return Workload("custom", B=B, Q=Q, M=M, D=D, shapes=tuple(tuple(s) for s in shapes), K=K,
                    dtype=dtype, ref=ref, sigma_px=sigma_px)
