"""Python binding of the MI355X MSDA library (``libmsda.so``, C ABI in include/msda.h).

Argument marshalling only: every step of the operator runs in the HIP kernels
of the library.  torch supplies device memory and the stream.  If the library
has not been built this module raises on first use; there is no fallback.

The functions keep the C names:
    msda_forward(value, spatial_shapes, level_start_index, sampling_locations,
                 attention_weights, out=None, stream=None) -> out
    msda_backward(value, spatial_shapes, level_start_index, sampling_locations,
                  attention_weights, grad_out, grad_value=None, grad_loc=None,
                  grad_attn=None, accum_dtype=None, workspace=None, stream=None)
                  -> (grad_value, grad_loc, grad_attn)
    msda_backward_workspace_bytes(dims, dtype, accum_dtype) -> int
    msda_status_string(status) -> str
    msda_last_error() -> str
Shapes follow chapter 1 of the msda-triton course ("The equation, term by
term"): value (B, S, M, D), spatial_shapes (L, 2) rows (H, W),
level_start_index (L,), sampling_locations (B, Q, M, L, K, 2),
attention_weights (B, Q, M, L, K), output (B, Q, M*D).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmsda.so")

MSDA_OK = 0
MSDA_FP32 = 0
MSDA_BF16 = 1
_DTYPES = {torch.float32: MSDA_FP32, torch.bfloat16: MSDA_BF16}


class MsdaDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("num_keys", ctypes.c_int64),
                ("num_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("num_levels", ctypes.c_int64), ("num_queries", ctypes.c_int64),
                ("num_points", ctypes.c_int64)]


class MsdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {msda_status_string(status)} ({msda_last_error()})")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmsda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m scale_deformable_attention_msda_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64p, dims_p = ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(MsdaDims)
    lib.msda_forward.argtypes = [vp, i64p, i64p, vp, vp, vp, dims_p, ctypes.c_int, vp]
    lib.msda_forward.restype = ctypes.c_int
    lib.msda_backward.argtypes = [vp, i64p, i64p, vp, vp, vp, vp, vp, vp, dims_p, ctypes.c_int,
                                  ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.msda_backward.restype = ctypes.c_int
    lib.msda_backward_workspace_bytes.argtypes = [dims_p, ctypes.c_int, ctypes.c_int]
    lib.msda_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.msda_status_string.argtypes = [ctypes.c_int]
    lib.msda_status_string.restype = ctypes.c_char_p
    lib.msda_last_error.argtypes = []
    lib.msda_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def msda_status_string(status: int) -> str:
    return load_library().msda_status_string(status).decode()


def msda_last_error() -> str:
    return load_library().msda_last_error().decode()


def _dims_of(value: torch.Tensor, spatial_shapes: torch.Tensor,
             sampling_locations: torch.Tensor) -> MsdaDims:
    B, S, M, D = value.shape
    L = spatial_shapes.shape[0]
    Q, K = sampling_locations.shape[1], sampling_locations.shape[4]
    return MsdaDims(B, S, M, D, L, Q, K)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _common(value, spatial_shapes, level_start_index, sampling_locations, attention_weights):
    if value.dtype not in _DTYPES:
        raise ValueError(f"value dtype {value.dtype} is not float32 or bfloat16")
    dt = value.dtype
    _check(value, "value")
    _check(spatial_shapes, "spatial_shapes", torch.int64)
    _check(level_start_index, "level_start_index", torch.int64)
    dims = _dims_of(value, spatial_shapes, sampling_locations)
    B, S, M, D, L, Q, K = (dims.batch, dims.num_keys, dims.num_heads, dims.head_dim,
                           dims.num_levels, dims.num_queries, dims.num_points)
    _check(sampling_locations, "sampling_locations", dt, (B, Q, M, L, K, 2))
    _check(attention_weights, "attention_weights", dt, (B, Q, M, L, K))
    return dims, dt


def msda_forward(value, spatial_shapes, level_start_index, sampling_locations,
                 attention_weights, out=None, stream=None):
    """out[B, Q, M*D] = MSDA(...) computed by the library's forward kernel."""
    dims, dt = _common(value, spatial_shapes, level_start_index, sampling_locations,
                       attention_weights)
    shape = (dims.batch, dims.num_queries, dims.num_heads * dims.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=dt, device=value.device)
    _check(out, "out", dt, shape)
    st = load_library().msda_forward(_ptr(value), _ptr(spatial_shapes), _ptr(level_start_index),
                                     _ptr(sampling_locations), _ptr(attention_weights),
                                     _ptr(out), ctypes.byref(dims), _DTYPES[dt], _stream(stream))
    if st != MSDA_OK:
        raise MsdaError(st, "msda_forward")
    return out


def msda_backward_workspace_bytes(dims: MsdaDims, dtype: int, accum_dtype: int) -> int:
    return int(load_library().msda_backward_workspace_bytes(ctypes.byref(dims), dtype,
                                                            accum_dtype))


def msda_backward(value, spatial_shapes, level_start_index, sampling_locations,
                  attention_weights, grad_out, grad_value=None, grad_loc=None, grad_attn=None,
                  accum_dtype=None, workspace=None, stream=None):
    """Gradients of <out, grad_out> w.r.t. value, sampling_locations, attention_weights.

    accum_dtype: torch.float32 (default) or torch.bfloat16 (packed-bf16 atomics, bf16 data
    only).  A bf16 call with an fp32 accumulator needs a workspace; one is allocated here
    when none is given."""
    dims, dt = _common(value, spatial_shapes, level_start_index, sampling_locations,
                       attention_weights)
    B, S, M, D, L, Q, K = (dims.batch, dims.num_keys, dims.num_heads, dims.head_dim,
                           dims.num_levels, dims.num_queries, dims.num_points)
    _check(grad_out, "grad_out", dt, (B, Q, M * D))
    acc = _DTYPES[accum_dtype if accum_dtype is not None else torch.float32]
    dev = value.device
    if grad_value is None:
        grad_value = torch.empty_like(value)
    if grad_loc is None:
        grad_loc = torch.empty_like(sampling_locations)
    if grad_attn is None:
        grad_attn = torch.empty_like(attention_weights)
    _check(grad_value, "grad_value", dt, value.shape)
    _check(grad_loc, "grad_loc", dt, sampling_locations.shape)
    _check(grad_attn, "grad_attn", dt, attention_weights.shape)
    need = msda_backward_workspace_bytes(dims, _DTYPES[dt], acc)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().msda_backward(
        _ptr(value), _ptr(spatial_shapes), _ptr(level_start_index), _ptr(sampling_locations),
        _ptr(attention_weights), _ptr(grad_out), _ptr(grad_value), _ptr(grad_loc),
        _ptr(grad_attn), ctypes.byref(dims), _DTYPES[dt], acc, _ptr(workspace), ws_bytes,
        _stream(stream))
    if st != MSDA_OK:
        raise MsdaError(st, "msda_backward")
    return grad_value, grad_loc, grad_attn
