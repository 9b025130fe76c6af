"""Layer-level use of the operator: the projections of a multi-scale deformable
attention layer (torch matmuls) around the library's "softmax"-method entry
points, with autograd.

Structure as the DeformOps page describes its layer (section "Multi-scale
deformable attention"): an embedding of `dim` channels split into `num_heads`
heads, `num_levels` feature levels and `num_points` points per level and
head; the layer takes queries, per-level reference points normalised to
[0, 1], the flattened value feature maps with their level shapes and starts,
and it asks the operator for the softmax of raw attention logits.  Sampling
locations are the reference point plus a learned offset in pixels of each
level, divided by that level's width (x) and height (y).

Only argument marshalling and autograd bookkeeping live here: the sampling,
the softmax and their gradients run in the library's kernels.
"""
from __future__ import annotations

import torch
from torch import nn

from . import msda_backward_softmax, msda_forward_softmax


class MSDASoftmaxFunction(torch.autograd.Function):
    """out = MSDA(value, ..., softmax(attention_logits)) with its backward.

    spatial_shapes_host: the level shapes on the host ([L, 2] int64 array-like),
    needed by the binned backward to plan its tiles.  scatter: how the backward
    forms grad_value, "binned" (a workspace, no atomics) or "atomic" (no
    workspace for fp32)."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start_index, sampling_locations,
                attention_logits, spatial_shapes_host, scatter="binned"):
        out = msda_forward_softmax(value, spatial_shapes, level_start_index, sampling_locations,
                                   attention_logits)
        ctx.save_for_backward(value, spatial_shapes, level_start_index, sampling_locations,
                              attention_logits)
        ctx.spatial_shapes_host = spatial_shapes_host
        ctx.scatter = scatter
        return out

    @staticmethod
    def backward(ctx, grad_out):
        value, shapes, starts, loc, logits = ctx.saved_tensors
        gv, gl, gz = msda_backward_softmax(value, shapes, starts, loc, logits,
                                           grad_out.contiguous(), scatter=ctx.scatter,
                                           spatial_shapes_host=ctx.spatial_shapes_host)
        return gv, None, None, gl, gz, None, None


def msda_softmax(value, spatial_shapes, level_start_index, sampling_locations, attention_logits,
                 spatial_shapes_host, scatter="binned"):
    """Differentiable softmax-method MSDA on the library's kernels."""
    return MSDASoftmaxFunction.apply(value, spatial_shapes, level_start_index,
                                     sampling_locations, attention_logits, spatial_shapes_host,
                                     scatter)


class MultiScaleDeformAttn(nn.Module):
    """value_proj -> MSDA (softmax method) -> output_proj, with the sampling
    offsets and attention logits predicted from the queries.

    `sampler` computes out[B, Q, M*D] from (value [B,S,M,D], spatial_shapes,
    level_start_index, sampling_locations, attention_logits,
    spatial_shapes_host); the default (None) is the library's operator, whose
    backward forms grad_value as `scatter` says.  Another sampler (a comparison
    composition) can be put in its place."""

    def __init__(self, dim: int = 256, num_heads: int = 8, num_levels: int = 4,
                 num_points: int = 4, sampler=None, scatter: str = "binned"):
        super().__init__()
        if dim % num_heads:
            raise ValueError(f"dim {dim} is not a multiple of num_heads {num_heads}")
        self.dim, self.num_heads = dim, num_heads
        self.num_levels, self.num_points = num_levels, num_points
        n = num_heads * num_levels * num_points
        self.value_proj = nn.Linear(dim, dim)
        self.sampling_offsets = nn.Linear(dim, 2 * n)
        self.attention_logits = nn.Linear(dim, n)
        self.output_proj = nn.Linear(dim, dim)
        self.sampler = sampler
        self.scatter = scatter

    def forward(self, query, reference, value, spatial_shapes, level_start_index,
                spatial_shapes_host=None):
        """query [B, Q, dim]; reference [B, Q, L, 2] normalised (x, y); value [B, S, dim];
        spatial_shapes [L, 2] int64 rows (H, W); level_start_index [L] int64."""
        B, Q, _ = query.shape
        S = value.shape[1]
        M, L, K = self.num_heads, self.num_levels, self.num_points
        D = self.dim // M
        if spatial_shapes_host is None:
            spatial_shapes_host = spatial_shapes.detach().cpu().numpy()
        v = self.value_proj(value).view(B, S, M, D)
        off = self.sampling_offsets(query).view(B, Q, M, L, K, 2)
        # offsets are in pixels of each level: x / W_l, y / H_l
        wh = spatial_shapes.flip(-1).to(off.dtype)
        loc = reference[:, :, None, :, None, :] + off / wh[None, None, None, :, None, :]
        logits = self.attention_logits(query).view(B, Q, M, L, K)
        if self.sampler is None:
            out = msda_softmax(v, spatial_shapes, level_start_index, loc.contiguous(),
                               logits.contiguous(), spatial_shapes_host, self.scatter)
        else:
            out = self.sampler(v, spatial_shapes, level_start_index, loc.contiguous(),
                               logits.contiguous(), spatial_shapes_host)
        return self.output_proj(out)
