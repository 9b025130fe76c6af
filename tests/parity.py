"""Helpers for the GPU-vs-oracle parity tests: upload, run both sides, compare.

Tolerances are the ones stated for this operator:
  forward fp32   rtol 1e-5, atol 1e-6
  backward fp32  rtol 1e-4, atol 1e-5  (grad_value order is set by atomics)
  bf16 paths     rtol 2e-2, atol 2e-2  (against the fp64 oracle on the same
                                        bf16-exact inputs)
  fp16 paths     rtol 2.5e-3, atol 2.5e-3  (the bf16 tolerance scaled by the
                                        ratio of unit roundoffs, 2^-11 / 2^-8)
An element passes when |gpu - oracle| <= atol + rtol * |oracle|.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import scale_deformable_attention_msda_amd as msda

TOL_FWD_FP32 = (1e-5, 1e-6)
TOL_BWD_FP32 = (1e-4, 1e-5)
TOL_BF16 = (2e-2, 2e-2)
TOL_FP16 = (2.5e-3, 2.5e-3)
TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}
HALF_TOL = {"bf16": TOL_BF16, "fp16": TOL_FP16}

FLOAT_KEYS = ("value", "sampling_locations", "attention_weights", "attention_logits", "grad_out")


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def upload(x: dict, device="cuda") -> dict:
    dt = TORCH_DTYPE[x["dtype"]]
    t = {k: torch.from_numpy(np.ascontiguousarray(x[k])).to(device).to(dt)
         for k in FLOAT_KEYS if k in x}
    t["spatial_shapes"] = torch.from_numpy(x["spatial_shapes"]).to(device)
    t["level_start_index"] = torch.from_numpy(x["level_start_index"]).to(device)
    return t


def operands(t: dict):
    return (t["value"], t["spatial_shapes"], t["level_start_index"], t["sampling_locations"],
            t["attention_weights"])


def run_gpu(x: dict, accum=None, stream=None, scatter="binned", gather="direct") -> dict:
    t = upload(x)
    out = msda.msda_forward(*operands(t), stream=stream, gather=gather,
                            spatial_shapes_host=x["spatial_shapes"])
    gv, gl, ga = msda.msda_backward(*operands(t), t["grad_out"], accum_dtype=accum, stream=stream,
                                    scatter=scatter, spatial_shapes_host=x["spatial_shapes"])
    torch.cuda.synchronize()
    return {k: v.double().cpu().numpy() for k, v in
            dict(out=out, grad_value=gv, grad_loc=gl, grad_attn=ga).items()}


def run_oracle(x: dict) -> dict:
    args = (x["value"], x["spatial_shapes"], x["level_start_index"], x["sampling_locations"],
            x["attention_weights"])
    out = oracle.forward(*args)
    gv, gl, ga = oracle.backward(*args, x["grad_out"])
    return dict(out=out, grad_value=gv, grad_loc=gl, grad_attn=ga)


def run_gpu_softmax(x: dict, accum=None, scatter="binned") -> dict:
    """The "softmax" method: msda_forward_softmax and msda_backward_softmax on the logits."""
    t = upload(x)
    ops = (t["value"], t["spatial_shapes"], t["level_start_index"], t["sampling_locations"],
           t["attention_logits"])
    out = msda.msda_forward_softmax(*ops)
    gv, gl, gz = msda.msda_backward_softmax(*ops, t["grad_out"], accum_dtype=accum,
                                            scatter=scatter,
                                            spatial_shapes_host=x["spatial_shapes"])
    torch.cuda.synchronize()
    return {k: v.double().cpu().numpy() for k, v in
            dict(out=out, grad_value=gv, grad_loc=gl, grad_logits=gz).items()}


def run_oracle_softmax(x: dict) -> dict:
    args = (x["value"], x["spatial_shapes"], x["level_start_index"], x["sampling_locations"],
            x["attention_logits"])
    out = oracle.forward_softmax(*args)
    gv, gl, gz = oracle.backward_softmax(*args, x["grad_out"])
    return dict(out=out, grad_value=gv, grad_loc=gl, grad_logits=gz)


def violations(got: np.ndarray, want: np.ndarray, rtol: float, atol: float):
    got = np.asarray(got, dtype=np.float64).ravel()
    want = np.asarray(want, dtype=np.float64).ravel()
    assert got.shape == want.shape
    err = np.abs(got - want)
    bound = atol + rtol * np.abs(want)
    bad = ~(err <= bound)  # NaN on either side counts as a violation
    return bad, err


def check(name: str, got, want, rtol: float, atol: float):
    bad, err = violations(got, want, rtol, atol)
    n = int(bad.sum())
    want_f = np.asarray(want).ravel()
    worst = int(np.argmax(np.where(np.isnan(err), np.inf, err))) if err.size else 0
    msg = (f"{name}: {n}/{err.size} outside atol {atol:g} + rtol {rtol:g}; max|err| "
           f"{np.nanmax(err) if err.size else 0:.3e} (oracle {want_f[worst] if err.size else 0:.4g})")
    say("  " + msg)
    assert n == 0, msg


def error_stats(got, want) -> dict:
    got = np.asarray(got, dtype=np.float64).ravel()
    want = np.asarray(want, dtype=np.float64).ravel()
    d = got - want
    return dict(max_abs=float(np.max(np.abs(d))),
                rel_l2=float(np.linalg.norm(d) / max(np.linalg.norm(want), 1e-300)),
                mean_bias=float(np.mean(d)))
