"""Python binding of the MI355X MSDA library (``libmsda.so``, C ABI in include/msda.h).

Argument marshalling only: every step of the operator runs in the HIP kernels
of the library.  torch supplies device memory and the stream.  If the library
has not been built this module raises on first use; there is no fallback.

The functions keep the C names:
    msda_forward(value, spatial_shapes, level_start_index, sampling_locations,
                 attention_weights, out=None, stream=None, gather="direct",
                 spatial_shapes_host=None, workspace=None) -> out
        (gather="binned" calls msda_forward_binned)
    msda_forward_binned_workspace_bytes(dims, dtype, spatial_shapes_host) -> int
    msda_backward(value, spatial_shapes, level_start_index, sampling_locations,
                  attention_weights, grad_out, grad_value=None, grad_loc=None,
                  grad_attn=None, accum_dtype=None, scatter="binned",
                  spatial_shapes_host=None, workspace=None, stream=None)
                  -> (grad_value, grad_loc, grad_attn)
    msda_backward_workspace_bytes(dims, dtype, accum_dtype, scatter,
                                  spatial_shapes_host) -> int
    msda_backward_flags(dims, dtype, accum_dtype, scatter, softmax_method,
                        spatial_shapes_host, workspace, stream=None) -> int
    msda_status_string(status) -> str
    msda_last_error() -> str
Measurement hooks (include/msda_bench.h): msda_profile_start / _select / _stop,
msda_microbench_run, msda_test_set_plan_wait_limit.
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
MSDA_FP16 = 2
MSDA_SCATTER_BINNED = 0
MSDA_SCATTER_ATOMIC = 1
_DTYPES = {torch.float32: MSDA_FP32, torch.bfloat16: MSDA_BF16, torch.float16: MSDA_FP16}
_SCATTER = {"binned": MSDA_SCATTER_BINNED, "atomic": MSDA_SCATTER_ATOMIC}
SIZE_MAX = 2 ** 64 - 1


class MsdaDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("num_keys", ctypes.c_int64),
                ("num_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("num_levels", ctypes.c_int64), ("num_queries", ctypes.c_int64),
                ("num_points", ctypes.c_int64)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("ms", ctypes.c_float)]


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
    lib.msda_forward_softmax.argtypes = lib.msda_forward.argtypes
    lib.msda_forward_softmax.restype = ctypes.c_int
    lib.msda_forward_binned.argtypes = [vp, i64p, i64p, vp, vp, vp, dims_p, ctypes.c_int, vp, vp,
                                        ctypes.c_size_t, vp]
    lib.msda_forward_binned.restype = ctypes.c_int
    lib.msda_forward_binned_reuse.argtypes = lib.msda_forward_binned.argtypes
    lib.msda_forward_binned_reuse.restype = ctypes.c_int
    lib.msda_forward_binned_workspace_bytes.argtypes = [dims_p, ctypes.c_int, vp]
    lib.msda_forward_binned_workspace_bytes.restype = ctypes.c_size_t
    lib.msda_backward.argtypes = [vp, i64p, i64p, vp, vp, vp, vp, vp, vp, dims_p, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_size_t, vp]
    lib.msda_backward.restype = ctypes.c_int
    lib.msda_backward_workspace_bytes.argtypes = [dims_p, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int, vp]
    lib.msda_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.msda_backward_softmax.argtypes = lib.msda_backward.argtypes
    lib.msda_backward_softmax.restype = ctypes.c_int
    lib.msda_backward_softmax_workspace_bytes.argtypes = lib.msda_backward_workspace_bytes.argtypes
    lib.msda_backward_softmax_workspace_bytes.restype = ctypes.c_size_t
    lib.msda_status_string.argtypes = [ctypes.c_int]
    lib.msda_status_string.restype = ctypes.c_char_p
    lib.msda_last_error.argtypes = []
    lib.msda_last_error.restype = ctypes.c_char_p
    lib.msda_profile_start.argtypes = [ctypes.c_int]
    lib.msda_profile_start.restype = ctypes.c_int
    lib.msda_profile_stop.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int]
    lib.msda_profile_stop.restype = ctypes.c_int
    lib.msda_profile_select.argtypes = [ctypes.c_char_p]
    lib.msda_profile_select.restype = None
    lib.msda_backward_flags.argtypes = [dims_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, vp, vp, ctypes.c_size_t, vp,
                                        ctypes.POINTER(ctypes.c_uint32)]
    lib.msda_backward_flags.restype = ctypes.c_int
    lib.msda_backward_noalloc.argtypes = lib.msda_backward.argtypes[:14] + [vp]
    lib.msda_backward_noalloc.restype = ctypes.c_int
    lib.msda_noalloc_scratch_bytes.argtypes = []
    lib.msda_noalloc_scratch_bytes.restype = ctypes.c_size_t
    # test hooks: bound where the library has them (a tuning variant built from
    # older sources may lack a newer hook; calling a missing one raises)
    for name, arg in (("msda_test_set_forward_schedule", ctypes.c_int),
                      ("msda_test_set_tile_wide_addressing", ctypes.c_int),
                      ("msda_test_set_plan_wait_limit", ctypes.c_uint32)):
        if hasattr(lib, name):
            getattr(lib, name).argtypes = [arg]
            getattr(lib, name).restype = None
    if hasattr(lib, "msda_test_tile_phase_clocks"):
        lib.msda_test_tile_phase_clocks.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.c_int]
        lib.msda_test_tile_phase_clocks.restype = ctypes.c_int
    lib.msda_microbench_run.argtypes = [ctypes.c_int, vp, ctypes.c_size_t, ctypes.c_size_t,
                                        ctypes.c_int, vp, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double)]
    lib.msda_microbench_run.restype = ctypes.c_int
    _lib = lib
    return lib


def msda_status_string(status: int) -> str:
    return load_library().msda_status_string(status).decode()


def msda_last_error() -> str:
    return load_library().msda_last_error().decode()


def msda_profile_start(capacity: int) -> None:
    """Time every kernel the library enqueues from this thread (HIP events on its stream)."""
    st = load_library().msda_profile_start(capacity)
    if st != MSDA_OK:
        raise MsdaError(st, "msda_profile_start")


def msda_profile_select(name: str | None) -> None:
    """Time only kernels of this name in later sessions (None: all kernels)."""
    load_library().msda_profile_select(None if name is None else name.encode())


def msda_profile_stop(max_records: int = 1 << 16) -> list:
    """End the session; return [(kernel name, milliseconds), ...] in launch order."""
    buf = (KernelTime * max_records)()
    n = load_library().msda_profile_stop(buf, max_records)
    if n < 0:
        raise RuntimeError("msda_profile_stop: a HIP event call failed")
    return [(buf[i].name.decode(), float(buf[i].ms)) for i in range(min(n, max_records))]


MSDA_BWD_SHAPES_MISMATCH = 1
MSDA_BWD_PLAN_EXPIRED = 2
MICROBENCH = {"read": 0, "copy": 1, "atomic_f32": 2, "atomic_pk_bf16": 3, "gather_global": 4,
              "gather_lds": 5, "lds_atomic_f32": 6}


FORWARD_SCHEDULE = {"auto": 0, "direct": 1, "window": 2}


def msda_test_set_forward_schedule(schedule: str) -> None:
    """Test hook: forward schedule of later calls on this thread ("auto", "direct" or
    "window")."""
    load_library().msda_test_set_forward_schedule(FORWARD_SCHEDULE[schedule])


def msda_test_set_tile_wide_addressing(wide: bool) -> None:
    """Test hook: later binned backward calls on this thread run the tile pass's 64-bit
    addressing path (True) or pick it by size (False, the default)."""
    load_library().msda_test_set_tile_wide_addressing(1 if wide else 0)


def msda_test_tile_phase_clocks(nblocks: int = 2048) -> list[list[int]]:
    """Diagnostic: per-block shader-clock sums of the last tile pass's phases,
    nblocks rows of 12 values (see msda_bench.h).  Raises unless the loaded library
    was built with -DMSDA_TILE_PHASE_CLOCKS."""
    buf = (ctypes.c_ulonglong * (nblocks * 12))()
    st = load_library().msda_test_tile_phase_clocks(buf, nblocks)
    if st != 0:
        raise MsdaError(st, "msda_test_tile_phase_clocks")
    return [list(buf[12 * b:12 * b + 12]) for b in range(nblocks)]


def msda_test_set_plan_wait_limit(polls: int) -> None:
    """Test hook: later binned backward plans on this thread give up waiting after `polls`."""
    load_library().msda_test_set_plan_wait_limit(polls)


def msda_microbench_run(kind: str, buf: torch.Tensor, span: int = 0, reps: int = 10,
                        stream=None) -> tuple[float, float]:
    """Run one memory-path microbenchmark on device buffer `buf` (overwritten);
    returns (milliseconds per launch, units per launch)."""
    _check(buf, "buf")
    ms, units = ctypes.c_double(), ctypes.c_double()
    rc = load_library().msda_microbench_run(MICROBENCH[kind], buf.data_ptr(),
                                            buf.numel() * buf.element_size(), span, reps,
                                            _stream(stream), ctypes.byref(ms), ctypes.byref(units))
    if rc != 0:
        raise RuntimeError(f"msda_microbench_run({kind!r}) returned {rc}")
    return ms.value, units.value


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


def _common(value, spatial_shapes, level_start_index, sampling_locations, attention_weights,
            weights_name="attention_weights"):
    if value.dtype not in _DTYPES:
        raise ValueError(f"value dtype {value.dtype} is not float32, bfloat16 or float16")
    dt = value.dtype
    _check(value, "value")
    _check(spatial_shapes, "spatial_shapes", torch.int64)
    _check(level_start_index, "level_start_index", torch.int64)
    dims = _dims_of(value, spatial_shapes, sampling_locations)
    B, S, M, D, L, Q, K = (dims.batch, dims.num_keys, dims.num_heads, dims.head_dim,
                           dims.num_levels, dims.num_queries, dims.num_points)
    _check(sampling_locations, "sampling_locations", dt, (B, Q, M, L, K, 2))
    _check(attention_weights, weights_name, dt, (B, Q, M, L, K))
    return dims, dt


def msda_forward_binned_workspace_bytes(dims: MsdaDims, dtype: int, spatial_shapes_host) -> int:
    """Workspace bytes msda_forward_binned needs; raises when it would reject the call."""
    import numpy as np

    host = np.ascontiguousarray(np.asarray(spatial_shapes_host, dtype=np.int64))
    n = int(load_library().msda_forward_binned_workspace_bytes(ctypes.byref(dims), dtype,
                                                                host.ctypes.data))
    if n == SIZE_MAX:
        raise ValueError(f"msda_forward_binned_workspace_bytes: {msda_last_error()}")
    return n


def msda_forward(value, spatial_shapes, level_start_index, sampling_locations,
                 attention_weights, out=None, stream=None, gather="direct",
                 spatial_shapes_host=None, workspace=None, reuse_order=False):
    """out[B, Q, M*D] = MSDA(...) computed by the library's forward kernels.

    gather: "direct" (default, msda_forward) or "binned" (msda_forward_binned: head-queries
    sorted by region, gathers from LDS-staged windows; needs the level shapes on the host,
    read from spatial_shapes when spatial_shapes_host is omitted, and a workspace, allocated
    here when none is given).  reuse_order (binned only): skip the sort and use the order an
    earlier binned call with the same sizes left in `workspace` (msda_forward_binned_reuse)."""
    dims, dt = _common(value, spatial_shapes, level_start_index, sampling_locations,
                       attention_weights)
    if gather not in ("binned", "direct"):
        raise ValueError(f"gather {gather!r} is not 'binned' or 'direct'")
    if reuse_order and gather != "binned":
        raise ValueError("reuse_order applies to the binned gather only")
    shape = (dims.batch, dims.num_queries, dims.num_heads * dims.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=dt, device=value.device)
    _check(out, "out", dt, shape)
    lib = load_library()
    args = (_ptr(value), _ptr(spatial_shapes), _ptr(level_start_index), _ptr(sampling_locations),
            _ptr(attention_weights), _ptr(out), ctypes.byref(dims), _DTYPES[dt])
    if gather == "direct":
        st = lib.msda_forward(*args, _stream(stream))
        if st != MSDA_OK:
            raise MsdaError(st, "msda_forward")
        return out
    host = _host_shapes(spatial_shapes, spatial_shapes_host)
    need = msda_forward_binned_workspace_bytes(dims, _DTYPES[dt], host)
    if reuse_order and workspace is None:
        raise ValueError("reuse_order needs the workspace of an earlier binned call")
    if need and workspace is None:
        workspace = _scratch(need, value.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = "msda_forward_binned_reuse" if reuse_order else "msda_forward_binned"
    st = getattr(lib, fn)(*args, host.ctypes.data, _ptr(workspace), ws_bytes, _stream(stream))
    if st != MSDA_OK:
        raise MsdaError(st, fn)
    return out


def msda_forward_softmax(value, spatial_shapes, level_start_index, sampling_locations,
                         attention_logits, out=None, stream=None):
    """out[B, Q, M*D] of the "softmax" method: the weights are the softmax of
    attention_logits over the L*K samples of each head-query, formed inside the kernel."""
    dims, dt = _common(value, spatial_shapes, level_start_index, sampling_locations,
                       attention_logits, "attention_logits")
    shape = (dims.batch, dims.num_queries, dims.num_heads * dims.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=dt, device=value.device)
    _check(out, "out", dt, shape)
    st = load_library().msda_forward_softmax(
        _ptr(value), _ptr(spatial_shapes), _ptr(level_start_index), _ptr(sampling_locations),
        _ptr(attention_logits), _ptr(out), ctypes.byref(dims), _DTYPES[dt], _stream(stream))
    if st != MSDA_OK:
        raise MsdaError(st, "msda_forward_softmax")
    return out


def _scratch(nbytes: int, device, stream) -> torch.Tensor:
    """A workspace the library uses only inside one call's enqueued work.

    It is allocated on the caller's current stream; when the kernels run on another
    stream, record_stream keeps the caching allocator from handing the block out again
    before that stream's work has finished."""
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None:
        s = stream if isinstance(stream, torch.cuda.Stream) else None
        cur = torch.cuda.current_stream(device)
        if s is None:
            s = torch.cuda.ExternalStream(_stream(stream), device=device)
        if s.cuda_stream != cur.cuda_stream:
            ws.record_stream(s)
    return ws


def msda_backward_flags(dims: MsdaDims, dtype: int, accum_dtype: int, scatter: int,
                        softmax_method: bool, spatial_shapes_host, workspace: torch.Tensor,
                        stream=None) -> int:
    """Device-side check flags a binned backward call left in `workspace` (waits for them):
    0 when its gradients are valid, else MSDA_BWD_* bits (the gradients are then NaN)."""
    import numpy as np

    host = np.ascontiguousarray(np.asarray(spatial_shapes_host, dtype=np.int64))
    flags = ctypes.c_uint32()
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load_library().msda_backward_flags(ctypes.byref(dims), dtype, accum_dtype, scatter,
                                            int(bool(softmax_method)), host.ctypes.data,
                                            workspace.data_ptr(), ws_bytes, _stream(stream),
                                            ctypes.byref(flags))
    if st != MSDA_OK:
        raise MsdaError(st, "msda_backward_flags")
    return int(flags.value)


def _host_shapes(spatial_shapes, spatial_shapes_host):
    """A contiguous int64 host array of the level shapes (kept alive by the caller)."""
    import numpy as np

    if spatial_shapes_host is None:
        spatial_shapes_host = spatial_shapes.detach().cpu()  # one device-to-host copy
    if isinstance(spatial_shapes_host, torch.Tensor):
        spatial_shapes_host = spatial_shapes_host.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(spatial_shapes_host, dtype=np.int64))


def _backward_ws_bytes(fn_name: str, dims: MsdaDims, dtype: int, accum_dtype: int, scatter: int,
                       spatial_shapes_host) -> int:
    host = None
    if spatial_shapes_host is not None:
        import numpy as np
        host = np.ascontiguousarray(np.asarray(spatial_shapes_host, dtype=np.int64))
    n = int(getattr(load_library(), fn_name)(
        ctypes.byref(dims), dtype, accum_dtype, scatter,
        None if host is None else host.ctypes.data))
    if n == SIZE_MAX:
        raise ValueError(f"{fn_name}: {msda_last_error()}")
    return n


def msda_backward_workspace_bytes(dims: MsdaDims, dtype: int, accum_dtype: int,
                                  scatter: int = MSDA_SCATTER_BINNED,
                                  spatial_shapes_host=None) -> int:
    """Workspace bytes msda_backward needs; raises when the call would be rejected."""
    return _backward_ws_bytes("msda_backward_workspace_bytes", dims, dtype, accum_dtype, scatter,
                              spatial_shapes_host)


def msda_backward_softmax_workspace_bytes(dims: MsdaDims, dtype: int, accum_dtype: int,
                                          scatter: int = MSDA_SCATTER_BINNED,
                                          spatial_shapes_host=None) -> int:
    """Workspace bytes msda_backward_softmax needs; raises when the call would be rejected."""
    return _backward_ws_bytes("msda_backward_softmax_workspace_bytes", dims, dtype, accum_dtype,
                              scatter, spatial_shapes_host)


def _backward(fn_name, value, spatial_shapes, level_start_index, sampling_locations, weights,
              grad_out, grad_value, grad_loc, grad_weights, accum_dtype, scatter,
              spatial_shapes_host, workspace, stream):
    dims, dt = _common(value, spatial_shapes, level_start_index, sampling_locations, weights,
                       "attention_logits" if fn_name.endswith("softmax") else "attention_weights")
    B, S, M, D, L, Q, K = (dims.batch, dims.num_keys, dims.num_heads, dims.head_dim,
                           dims.num_levels, dims.num_queries, dims.num_points)
    _check(grad_out, "grad_out", dt, (B, Q, M * D))
    acc = _DTYPES[accum_dtype if accum_dtype is not None else torch.float32]
    sc = _SCATTER[scatter]
    host = _host_shapes(spatial_shapes, spatial_shapes_host) if sc == MSDA_SCATTER_BINNED else None
    dev = value.device
    if grad_value is None:
        grad_value = torch.empty_like(value)
    if grad_loc is None:
        grad_loc = torch.empty_like(sampling_locations)
    if grad_weights is None:
        grad_weights = torch.empty_like(weights)
    _check(grad_value, "grad_value", dt, value.shape)
    _check(grad_loc, "grad_loc", dt, sampling_locations.shape)
    _check(grad_weights, "grad of the weights", dt, weights.shape)
    need = _backward_ws_bytes(fn_name + "_workspace_bytes", dims, _DTYPES[dt], acc, sc, host)
    if need and workspace is None:
        workspace = _scratch(need, dev, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = getattr(load_library(), fn_name)(
        _ptr(value), _ptr(spatial_shapes), _ptr(level_start_index), _ptr(sampling_locations),
        _ptr(weights), _ptr(grad_out), _ptr(grad_value), _ptr(grad_loc),
        _ptr(grad_weights), ctypes.byref(dims), _DTYPES[dt], acc, sc,
        None if host is None else host.ctypes.data, _ptr(workspace), ws_bytes, _stream(stream))
    if st != MSDA_OK:
        raise MsdaError(st, fn_name)
    return grad_value, grad_loc, grad_weights


def msda_backward(value, spatial_shapes, level_start_index, sampling_locations,
                  attention_weights, grad_out, grad_value=None, grad_loc=None, grad_attn=None,
                  accum_dtype=None, scatter="binned", spatial_shapes_host=None, workspace=None,
                  stream=None):
    """Gradients of <out, grad_out> w.r.t. value, sampling_locations, attention_weights.

    scatter: "binned" (default; destination-sorted, LDS accumulation, fp32) or "atomic"
    (device-scope atomics).  accum_dtype: torch.float32 (default) or the data type
    (atomic scatter of bf16 or fp16 data only: packed two-element atomics).  spatial_shapes_host: the
    level shapes on the host (array-like [L, 2]); read from spatial_shapes when omitted.
    A workspace is allocated here when none is given."""
    return _backward("msda_backward", value, spatial_shapes, level_start_index,
                     sampling_locations, attention_weights, grad_out, grad_value, grad_loc,
                     grad_attn, accum_dtype, scatter, spatial_shapes_host, workspace, stream)


def msda_noalloc_scratch_bytes() -> int:
    return int(load_library().msda_noalloc_scratch_bytes())


def msda_backward_noalloc(value, spatial_shapes, level_start_index, sampling_locations,
                          attention_weights, grad_out, grad_value, grad_loc, grad_attn,
                          accum_dtype=None, scatter="binned", spatial_shapes_host=None,
                          stream=None):
    """msda_backward without a workspace argument: the library takes it from its static
    per-GPU scratch array (msda_noalloc_scratch_bytes()).  The outputs must be given; no
    device memory is allocated here or in the library.  Calls overlapping on one GPU race."""
    dims, dt = _common(value, spatial_shapes, level_start_index, sampling_locations,
                       attention_weights)
    B, Q, M, D = dims.batch, dims.num_queries, dims.num_heads, dims.head_dim
    _check(grad_out, "grad_out", dt, (B, Q, M * D))
    _check(grad_value, "grad_value", dt, value.shape)
    _check(grad_loc, "grad_loc", dt, sampling_locations.shape)
    _check(grad_attn, "grad_attn", dt, attention_weights.shape)
    acc = _DTYPES[accum_dtype if accum_dtype is not None else torch.float32]
    sc = _SCATTER[scatter]
    host = _host_shapes(spatial_shapes, spatial_shapes_host) if sc == MSDA_SCATTER_BINNED else None
    st = load_library().msda_backward_noalloc(
        _ptr(value), _ptr(spatial_shapes), _ptr(level_start_index), _ptr(sampling_locations),
        _ptr(attention_weights), _ptr(grad_out), _ptr(grad_value), _ptr(grad_loc),
        _ptr(grad_attn), ctypes.byref(dims), _DTYPES[dt], acc, sc,
        None if host is None else host.ctypes.data, _stream(stream))
    if st != MSDA_OK:
        raise MsdaError(st, "msda_backward_noalloc")
    return grad_value, grad_loc, grad_attn


def msda_backward_softmax(value, spatial_shapes, level_start_index, sampling_locations,
                          attention_logits, grad_out, grad_value=None, grad_loc=None,
                          grad_logits=None, accum_dtype=None, scatter="binned",
                          spatial_shapes_host=None, workspace=None, stream=None):
    """Gradients of <out, grad_out> for the "softmax" method (weights = softmax of the
    logits over the L*K samples of each head-query) w.r.t. value, sampling_locations and
    attention_logits.  Arguments as for msda_backward."""
    return _backward("msda_backward_softmax", value, spatial_shapes, level_start_index,
                     sampling_locations, attention_logits, grad_out, grad_value, grad_loc,
                     grad_logits, accum_dtype, scatter, spatial_shapes_host, workspace, stream)
