"""Plain fp64 CPU oracle for the MSDA core operator (forward and gradients).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
and its Python binding never import, call or link it.

The arithmetic lives in ``msda_oracle.c`` (plain C, fp64, OpenMP over
independent outer loops); this module only builds it with gcc, converts the
operands to contiguous fp64 / int64 arrays (exact upcasts from fp32 or bf16)
and calls it through ctypes.  What it computes, and where the pages define it,
is stated in the C file: chapter 1 of the msda-triton course ("Deformable
attention, from scratch"), sections "The equation, term by term" (the
attention-weighted sum of level samples) and "Bilinear interpolation: reading
between the pixels" (the tent-weighted pixels around a point); the gradients
are derived there by hand.

Every function of the oracle is pinned by ``tests/test_oracle_pins.py``
(brute-force tent sums, closed forms, library routines, finite differences).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "msda_oracle.c")
LIB_PATH = os.path.join(_HERE, "libmsda_oracle.so")

_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build(source: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i64arr(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(typ)


def _dims(value, spatial_shapes, sampling_locations):
    B, S, M, D = value.shape
    L = spatial_shapes.shape[0]
    Bl, Q, Ml, Ll, K, two = sampling_locations.shape
    if (Bl, Ml, Ll, two) != (B, M, L, 2):
        raise ValueError("sampling_locations shape does not match value / spatial_shapes")
    return B, S, M, D, L, Q, K


class Oracle:
    """ctypes front of one compiled copy of ``msda_oracle.c``."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        common = [_f64p, _i64p, _i64p, _f64p, _f64p]
        dims = [_i64] * 7
        lib.msda_oracle_forward.argtypes = common + [_f64p] + dims
        lib.msda_oracle_forward.restype = None
        lib.msda_oracle_backward.argtypes = common + [_f64p, _f64p, _f64p, _f64p] + dims
        lib.msda_oracle_backward.restype = None
        lib.msda_oracle_threads.argtypes = []
        lib.msda_oracle_threads.restype = ctypes.c_int
        lib.msda_oracle_softmax.argtypes = [_f64p, _f64p, _i64, _i64]
        lib.msda_oracle_softmax.restype = None
        lib.msda_oracle_softmax_backward.argtypes = [_f64p, _f64p, _f64p, _i64, _i64]
        lib.msda_oracle_softmax_backward.restype = None
        self._lib = lib

    def threads(self) -> int:
        """OpenMP threads the oracle's loops run on."""
        return int(self._lib.msda_oracle_threads())

    def forward(self, value, spatial_shapes, level_start_index, sampling_locations,
                attention_weights):
        """Return out[B, Q, M*D] in fp64."""
        value, loc, attn = _f64(value), _f64(sampling_locations), _f64(attention_weights)
        shapes, starts = _i64arr(spatial_shapes), _i64arr(level_start_index)
        B, S, M, D, L, Q, K = _dims(value, shapes, loc)
        if attn.shape != (B, Q, M, L, K):
            raise ValueError("attention_weights shape mismatch")
        out = np.zeros((B, Q, M * D), dtype=np.float64)
        self._lib.msda_oracle_forward(_ptr(value, _f64p), _ptr(shapes, _i64p),
                                      _ptr(starts, _i64p), _ptr(loc, _f64p), _ptr(attn, _f64p),
                                      _ptr(out, _f64p), B, S, M, D, L, Q, K)
        return out

    def backward(self, value, spatial_shapes, level_start_index, sampling_locations,
                 attention_weights, grad_out):
        """Return (grad_value[B,S,M,D], grad_loc[B,Q,M,L,K,2], grad_attn[B,Q,M,L,K]), fp64."""
        value, loc, attn = _f64(value), _f64(sampling_locations), _f64(attention_weights)
        shapes, starts = _i64arr(spatial_shapes), _i64arr(level_start_index)
        B, S, M, D, L, Q, K = _dims(value, shapes, loc)
        g = _f64(grad_out).reshape(B, Q, M * D)
        if attn.shape != (B, Q, M, L, K):
            raise ValueError("attention_weights shape mismatch")
        grad_value = np.empty_like(value)
        grad_loc = np.empty_like(loc)
        grad_attn = np.empty_like(attn)
        self._lib.msda_oracle_backward(_ptr(value, _f64p), _ptr(shapes, _i64p),
                                       _ptr(starts, _i64p), _ptr(loc, _f64p), _ptr(attn, _f64p),
                                       _ptr(g, _f64p), _ptr(grad_value, _f64p),
                                       _ptr(grad_loc, _f64p), _ptr(grad_attn, _f64p),
                                       B, S, M, D, L, Q, K)
        return grad_value, grad_loc, grad_attn


    def softmax(self, logits):
        """Attention weights from raw logits [B,Q,M,L,K]: softmax over the L*K
        points of every (b, q, m) ("softmax" method), fp64."""
        z = _f64(logits)
        if z.ndim != 5:
            raise ValueError("logits must be [B, Q, M, L, K]")
        a = np.empty_like(z)
        lk = z.shape[3] * z.shape[4]
        self._lib.msda_oracle_softmax(_ptr(z, _f64p), _ptr(a, _f64p), z.size // lk, lk)
        return a

    def softmax_backward(self, weights, grad_weights):
        """grad_logits from the softmax's weights and dLoss/dweights, fp64."""
        a, ga = _f64(weights), _f64(grad_weights)
        if a.shape != ga.shape or a.ndim != 5:
            raise ValueError("weights and grad_weights must both be [B, Q, M, L, K]")
        out = np.empty_like(a)
        lk = a.shape[3] * a.shape[4]
        self._lib.msda_oracle_softmax_backward(_ptr(a, _f64p), _ptr(ga, _f64p),
                                               _ptr(out, _f64p), a.size // lk, lk)
        return out

    def forward_softmax(self, value, spatial_shapes, level_start_index, sampling_locations,
                        attention_logits):
        """The forward with weights = softmax(attention_logits)."""
        return self.forward(value, spatial_shapes, level_start_index, sampling_locations,
                            self.softmax(attention_logits))

    def backward_softmax(self, value, spatial_shapes, level_start_index, sampling_locations,
                         attention_logits, grad_out):
        """(grad_value, grad_loc, grad_logits) of the forward with softmax weights."""
        a = self.softmax(attention_logits)
        gv, gl, ga = self.backward(value, spatial_shapes, level_start_index, sampling_locations,
                                   a, grad_out)
        return gv, gl, self.softmax_backward(a, ga)


_default = None


def default() -> Oracle:
    """The oracle built from ``msda_oracle.c`` (built on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def forward(*args):
    return default().forward(*args)


def backward(*args):
    return default().backward(*args)


def forward_softmax(*args):
    return default().forward_softmax(*args)


def backward_softmax(*args):
    return default().backward_softmax(*args)
