"""The C-ABI library on the host: it loads, exports every symbol include/*.h
declares, and rejects bad arguments with a status code before any launch.
No call here reaches a kernel, so these run without a GPU."""
import ctypes
import os
import re

import pytest

import scale_deformable_attention_msda_amd as msda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msda.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(msda.LIB_PATH):
        from scale_deformable_attention_msda_amd import build
        build.build()
    return msda.load_library()


def declared_functions(headers=HEADERS):
    names = set()
    for h in headers:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(msda_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("msda_forward", "msda_forward_binned", "msda_forward_binned_workspace_bytes",
              "msda_forward_softmax", "msda_backward", "msda_backward_workspace_bytes",
              "msda_backward_softmax", "msda_backward_softmax_workspace_bytes",
              "msda_status_string", "msda_last_error", "msda_backward_flags"):
        assert n in declared_functions([HEADER])
    for n in ("msda_profile_start", "msda_profile_stop", "msda_profile_select",
              "msda_microbench_run", "msda_test_set_plan_wait_limit"):
        assert n in names and n not in declared_functions([HEADER])


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_phase_clocks_need_the_diagnostic_build(lib):
    """The default library records no tile-pass phase clocks: the call reports
    MSDA_ERR_UNSUPPORTED without touching a device, and checks its arguments first."""
    null_pointer, invalid_dims, unsupported = 1, 2, 3  # msda_status in include/msda.h
    buf = (ctypes.c_ulonglong * 12)()
    assert lib.msda_test_tile_phase_clocks(buf, 1) == unsupported
    assert lib.msda_test_tile_phase_clocks(None, 1) == null_pointer
    assert lib.msda_test_tile_phase_clocks(buf, 4096) == invalid_dims
    with pytest.raises(msda.MsdaError):
        msda.msda_test_tile_phase_clocks(1)


def test_status_strings(lib):
    for code in range(7):
        assert msda.msda_status_string(code).startswith("MSDA_")
    assert "unknown" in msda.msda_status_string(99)


def dims(B=1, S=80, M=2, D=8, L=2, Q=16, K=2):
    return msda.MsdaDims(B, S, M, D, L, Q, K)


FAKE = 0x10000  # a 64 KiB-aligned non-null address; never dereferenced by a rejected call


def fwd(lib, d, dtype=0, value=FAKE, shapes=FAKE, starts=FAKE, loc=FAKE, attn=FAKE, out=FAKE):
    return lib.msda_forward(value, shapes, starts, loc, attn, out,
                            None if d is None else ctypes.byref(d), dtype, None)


def fwd_binned(lib, d, dtype=0, shapes_host=None, ws=None, ws_bytes=0):
    return lib.msda_forward_binned(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), dtype,
                                   shapes_host, ws, ws_bytes, None)


SHAPES = (ctypes.c_int64 * 4)(8, 8, 4, 4)  # host copy of [[8, 8], [4, 4]]
PYRAMID = (ctypes.c_int64 * 8)(100, 167, 50, 84, 25, 42, 13, 21)  # the 4-level encoder pyramid
ENCODER = dict(B=2, S=22223, M=8, D=32, L=4, Q=22223, K=4)
SIZE_MAX = 2 ** 64 - 1


def fwd_ws(lib, d, dtype=0, shapes_host=None):
    return lib.msda_forward_binned_workspace_bytes(ctypes.byref(d), dtype, shapes_host)


def bwd(lib, d, dtype=0, acc=0, scatter=1, shapes_host=None, ws=None, ws_bytes=0, **p):
    v = {k: p.get(k, FAKE) for k in ("value", "shapes", "starts", "loc", "attn", "gout", "gv",
                                     "gl", "ga")}
    return lib.msda_backward(v["value"], v["shapes"], v["starts"], v["loc"], v["attn"], v["gout"],
                             v["gv"], v["gl"], v["ga"], None if d is None else ctypes.byref(d),
                             dtype, acc, scatter, shapes_host, ws, ws_bytes, None)


def ws_bytes(lib, d, dtype=0, acc=0, scatter=0, shapes_host=None):
    return lib.msda_backward_workspace_bytes(ctypes.byref(d), dtype, acc, scatter, shapes_host)


def test_binned_forward_workspace_sizes(lib):
    # one query per pyramid pixel: the binned gather plans it and needs a sort buffer
    need = fwd_ws(lib, dims(**ENCODER), 0, PYRAMID)
    assert 8 * 2 * 8 * 22223 <= need < 64 << 20
    assert fwd_ws(lib, dims(**ENCODER), 1, PYRAMID) > 0                       # bf16, 64-byte rows
    assert fwd_ws(lib, dims(**ENCODER), 2, PYRAMID) > 0                       # fp16, 64-byte rows
    assert fwd_ws(lib, dims(**ENCODER), 0, None) == SIZE_MAX                  # needs host shapes
    assert "spatial_shapes_host" in msda.msda_last_error()
    for bad in (dict(Q=300), dict(D=8), dict(K=9)):  # few queries, 32-byte rows, K > 8
        assert fwd_ws(lib, dims(**dict(ENCODER, **bad)), 0, PYRAMID) == SIZE_MAX
        assert "binned forward" in msda.msda_last_error()
    assert fwd_ws(lib, dims(D=12), 0, SHAPES) == SIZE_MAX


def test_binned_forward_rejections(lib):
    d = dims(**ENCODER)
    need = fwd_ws(lib, d, 0, PYRAMID)
    assert fwd_binned(lib, d, shapes_host=PYRAMID) == 5
    assert "workspace" in msda.msda_last_error()
    assert fwd_binned(lib, d, shapes_host=PYRAMID, ws=FAKE, ws_bytes=need - 1) == 5
    assert fwd_binned(lib, d, shapes_host=PYRAMID, ws=FAKE + 4, ws_bytes=need) == 4
    assert fwd_binned(lib, d, shapes_host=None, ws=FAKE, ws_bytes=need) == 1
    assert fwd_binned(lib, dims(**dict(ENCODER, Q=300)), shapes_host=PYRAMID, ws=FAKE,
                      ws_bytes=need) == 3


@pytest.mark.parametrize("kwargs,code", [
    (dict(D=12), 3), (dict(D=128), 3), (dict(L=0), 2), (dict(K=0), 2), (dict(L=17), 3),
    (dict(K=33), 3), (dict(L=8, K=9), 3), (dict(B=-1), 2), (dict(Q=-1), 2), (dict(S=0), 2),
    (dict(M=0), 2), (dict(S=1 << 58, M=8, D=64), 2), (dict(S=1 << 22, M=16, D=64), 3),
])
def test_forward_rejects_bad_dims(lib, kwargs, code):
    assert fwd(lib, dims(**kwargs)) == code
    assert msda.msda_last_error() != ""


def test_forward_rejects_bad_pointers_and_dtype(lib):
    assert fwd(lib, None) == 1
    assert fwd(lib, dims(), value=None) == 1
    assert fwd(lib, dims(), out=None) == 1
    assert fwd(lib, dims(), loc=FAKE + 4) == 4
    assert fwd(lib, dims(), value=FAKE + 8) == 4
    assert fwd(lib, dims(), dtype=3) == 3
    assert "dtype" in msda.msda_last_error()


def test_empty_forward_is_ok_without_launch(lib):
    # Q = 0: nothing to compute, the optional pointers may be NULL
    assert fwd(lib, dims(Q=0), loc=None, attn=None, out=None) == 0
    assert fwd(lib, dims(B=0), loc=None, attn=None, out=None) == 0


def test_backward_rejections_atomic(lib):
    assert bwd(lib, dims(), dtype=0, acc=1) == 3            # fp32 data needs fp32 accum
    assert bwd(lib, dims(), dtype=1, acc=0) == 5            # bf16 + fp32 accum needs workspace
    need = ws_bytes(lib, dims(), 1, 0, scatter=1)
    assert need == 1 * 80 * 2 * 8 * 4
    assert bwd(lib, dims(), dtype=1, acc=0, ws=FAKE, ws_bytes=need - 1) == 5
    assert bwd(lib, dims(), dtype=1, acc=0, ws=FAKE + 4, ws_bytes=need) == 4
    assert bwd(lib, dims(), gv=None) == 1
    assert bwd(lib, dims(), acc=7) == 3
    assert bwd(lib, dims(), scatter=5) == 3
    assert ws_bytes(lib, dims(), 0, 0, scatter=1) == 0
    assert ws_bytes(lib, dims(), 1, 1, scatter=1) == 0
    assert lib.msda_backward_workspace_bytes(None, 1, 0, 1, None) == 2 ** 64 - 1


def test_backward_rejections_binned(lib):
    assert bwd(lib, dims(), scatter=0) == 1                  # needs the host shapes
    assert "spatial_shapes_host" in msda.msda_last_error()
    assert bwd(lib, dims(), scatter=0, acc=1, dtype=1, shapes_host=SHAPES) == 3
    need = ws_bytes(lib, dims(), 0, 0, scatter=0, shapes_host=SHAPES)
    assert 0 < need < 1 << 24
    assert bwd(lib, dims(), scatter=0, shapes_host=SHAPES, ws=FAKE, ws_bytes=need - 1) == 5
    assert bwd(lib, dims(), scatter=0, shapes_host=SHAPES, ws=None, ws_bytes=need) == 5
    bad = (ctypes.c_int64 * 4)(8, 0, 4, 4)
    assert bwd(lib, dims(), scatter=0, shapes_host=bad) == 3
    too_big = (ctypes.c_int64 * 4)(16, 16, 4, 4)          # 272 pixels > num_keys = 80
    assert bwd(lib, dims(), scatter=0, shapes_host=too_big) == 3
    assert ws_bytes(lib, dims(), 0, 0, scatter=0, shapes_host=bad) == 2 ** 64 - 1
    # no samples: nothing to plan, no workspace
    assert ws_bytes(lib, dims(Q=0), 0, 0, scatter=0, shapes_host=None) == 0


def test_last_error_is_cleared_by_a_good_call(lib):
    assert fwd(lib, dims(D=12)) == 3
    assert msda.msda_last_error() != ""
    assert fwd(lib, dims(Q=0), loc=None, attn=None, out=None) == 0
    assert msda.msda_last_error() == ""


def fwd_softmax(lib, d, dtype=0, value=FAKE, logits=FAKE, out=FAKE):
    return lib.msda_forward_softmax(value, FAKE, FAKE, FAKE, logits, out,
                                    None if d is None else ctypes.byref(d), dtype, None)


def bwd_softmax(lib, d, dtype=0, acc=0, scatter=1, shapes_host=None, ws=None, ws_bytes=0,
                logits=FAKE, grad_logits=FAKE):
    return lib.msda_backward_softmax(FAKE, FAKE, FAKE, FAKE, logits, FAKE, FAKE, FAKE,
                                     grad_logits, ctypes.byref(d), dtype, acc, scatter,
                                     shapes_host, ws, ws_bytes, None)


def softmax_ws_bytes(lib, d, dtype=0, acc=0, scatter=1, shapes_host=None):
    return lib.msda_backward_softmax_workspace_bytes(ctypes.byref(d), dtype, acc, scatter,
                                                     shapes_host)


def test_softmax_forward_rejections(lib):
    assert fwd_softmax(lib, None) == 1
    assert fwd_softmax(lib, dims(D=12)) == 3
    assert fwd_softmax(lib, dims(L=8, K=9)) == 3
    assert fwd_softmax(lib, dims(), logits=None) == 1
    assert "attention_logits" in msda.msda_last_error()
    assert fwd_softmax(lib, dims(), logits=FAKE + 4) == 4
    assert fwd_softmax(lib, dims(), dtype=3) == 3
    assert fwd_softmax(lib, dims(Q=0), logits=None, out=None) == 0
    assert msda.msda_last_error() == ""


def test_softmax_backward_workspace_sizes(lib):
    # the weights image (B*Q*M*L*K elements rounded up to 256 bytes) ahead of the scatter's part
    d = dims()                                                   # 1*16*2*2*2 = 128 samples
    assert softmax_ws_bytes(lib, d, 0, 0, 1) == 512              # fp32, atomic: 512 + 0
    assert softmax_ws_bytes(lib, d, 1, 1, 1) == 256              # bf16 data, bf16 accum
    assert softmax_ws_bytes(lib, d, 1, 0, 1) == 256 + ws_bytes(lib, d, 1, 0, scatter=1)
    # binned with L*K = 4: the scatter pass forms the weights, no image
    binned = ws_bytes(lib, d, 0, 0, scatter=0, shapes_host=SHAPES)
    assert softmax_ws_bytes(lib, d, 0, 0, 0, SHAPES) == binned
    # binned with L*K = 6: the image again (1*16*2*2*3 * 4 bytes = 768)
    d6 = dims(K=3)
    binned6 = ws_bytes(lib, d6, 0, 0, scatter=0, shapes_host=SHAPES)
    assert softmax_ws_bytes(lib, d6, 0, 0, 0, SHAPES) == 768 + binned6
    assert softmax_ws_bytes(lib, dims(Q=3), 0, 0, 1) == 256      # 3*2*4*4 = 96 bytes, rounded
    assert softmax_ws_bytes(lib, dims(Q=0), 0, 0, 0, None) == 0
    assert softmax_ws_bytes(lib, d, 0, 0, 0, None) == SIZE_MAX   # binned needs host shapes
    assert softmax_ws_bytes(lib, d, 0, 1, 1) == SIZE_MAX         # fp32 data, bf16 accum


def test_softmax_backward_rejections(lib):
    d = dims()
    need = softmax_ws_bytes(lib, d, 0, 0, 1)
    assert bwd_softmax(lib, d) == 5                              # the weights need workspace
    assert "softmax backward" in msda.msda_last_error()
    assert bwd_softmax(lib, d, ws=FAKE, ws_bytes=need - 1) == 5
    assert bwd_softmax(lib, d, ws=FAKE + 4, ws_bytes=need) == 4
    assert bwd_softmax(lib, d, ws=FAKE, ws_bytes=need, grad_logits=None) == 1
    assert "grad_logits" in msda.msda_last_error()
    assert bwd_softmax(lib, d, ws=FAKE, ws_bytes=need, logits=None) == 1
    assert "attention_logits" in msda.msda_last_error()
    assert bwd_softmax(lib, d, scatter=0, ws=FAKE, ws_bytes=need) == 1
    assert bwd_softmax(lib, d, acc=1) == 3
    assert bwd_softmax(lib, dims(D=12)) == 3


def test_fp16_accumulators(lib):
    # FP16 data: the atomic scatter accumulates in FP32 (workspace) or FP16 (packed atomics)
    assert ws_bytes(lib, dims(), 2, 0, scatter=1) == 1 * 80 * 2 * 8 * 4
    assert ws_bytes(lib, dims(), 2, 2, scatter=1) == 0
    assert ws_bytes(lib, dims(), 2, 1, scatter=1) == SIZE_MAX      # BF16 accumulator, FP16 data
    assert "accumulates in FP32 or in the data type" in msda.msda_last_error()
    assert ws_bytes(lib, dims(), 1, 2, scatter=1) == SIZE_MAX      # FP16 accumulator, BF16 data
    assert bwd(lib, dims(), dtype=2, acc=0) == 5                   # needs the fp32 workspace
    assert bwd(lib, dims(), dtype=2, acc=2, scatter=0, shapes_host=SHAPES) == 3  # binned: fp32
    assert ws_bytes(lib, dims(), 2, 0, scatter=0, shapes_host=SHAPES) > 0
    assert bwd(lib, dims(), dtype=0, acc=2) == 3                   # FP32 data, FP16 accumulator


def fwd_reuse(lib, d, dtype=0, shapes_host=None, ws=None, ws_bytes=0):
    return lib.msda_forward_binned_reuse(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d),
                                         dtype, shapes_host, ws, ws_bytes, None)


def test_binned_forward_reuse_rejections(lib):
    d = dims(**ENCODER)
    need = fwd_ws(lib, d, 0, PYRAMID)
    assert fwd_reuse(lib, d, shapes_host=PYRAMID) == 5                  # needs the workspace
    assert fwd_reuse(lib, d, shapes_host=PYRAMID, ws=FAKE + 4, ws_bytes=need) == 4
    assert fwd_reuse(lib, d, shapes_host=None, ws=FAKE, ws_bytes=need) == 1
    # five 260 MB batch images (48 heads of 64 channels): more than one launch, so
    # no single order to reuse
    big = msda.MsdaDims(5, 22223, 48, 64, 4, 22223, 4)
    big_need = fwd_ws(lib, big, 0, PYRAMID)
    assert big_need != SIZE_MAX, msda.msda_last_error()
    assert fwd_reuse(lib, big, shapes_host=PYRAMID, ws=FAKE, ws_bytes=big_need) == 3
    assert "one launch" in msda.msda_last_error()


def test_backward_flags_host_side(lib):
    """msda_backward_flags: argument checks, and no device access for calls without
    device checks (atomic scatter, no samples)."""
    flags = ctypes.c_uint32(7)
    shapes = (ctypes.c_int64 * 4)(8, 8, 4, 4)
    dims = msda.MsdaDims(1, 80, 2, 8, 2, 16, 2)
    st = lib.msda_backward_flags(ctypes.byref(dims), msda.MSDA_FP32, msda.MSDA_FP32,
                                 msda.MSDA_SCATTER_ATOMIC, 0, shapes, None, 0, None,
                                 ctypes.byref(flags))
    assert st == msda.MSDA_OK and flags.value == 0
    empty = msda.MsdaDims(1, 80, 2, 8, 2, 0, 2)
    flags.value = 7
    st = lib.msda_backward_flags(ctypes.byref(empty), msda.MSDA_FP32, msda.MSDA_FP32,
                                 msda.MSDA_SCATTER_BINNED, 0, shapes, None, 0, None,
                                 ctypes.byref(flags))
    assert st == msda.MSDA_OK and flags.value == 0
    # a binned call with samples needs its workspace
    st = lib.msda_backward_flags(ctypes.byref(dims), msda.MSDA_FP32, msda.MSDA_FP32,
                                 msda.MSDA_SCATTER_BINNED, 0, shapes, None, 0, None,
                                 ctypes.byref(flags))
    assert st == 5  # MSDA_ERR_WORKSPACE
    st = lib.msda_backward_flags(ctypes.byref(dims), msda.MSDA_FP32, msda.MSDA_FP32,
                                 msda.MSDA_SCATTER_BINNED, 0, shapes, None, 0, None, None)
    assert st == 1  # MSDA_ERR_NULL_POINTER


def test_microbench_rejects_bad_arguments(lib):
    ms, units = ctypes.c_double(), ctypes.c_double()
    # NULL buffer, too small, bad kind: rejected before any launch
    assert lib.msda_microbench_run(0, None, 1 << 21, 0, 1, None, ctypes.byref(ms),
                                   ctypes.byref(units)) == 1
    assert lib.msda_microbench_run(0, 256, 1024, 0, 1, None, ctypes.byref(ms),
                                   ctypes.byref(units)) == 1
    assert lib.msda_microbench_run(0, 256, 1 << 21, 0, 0, None, ctypes.byref(ms),
                                   ctypes.byref(units)) == 1
