"""Helpers for the GPU parity tests: moving generated inputs to the device
and the float-comparison rule max|err| <= tau * RMS(ref)."""
import numpy as np
import torch

import moe_synth as synth

TAU = {"bf16": 2e-2, "f32": 1e-4}


def to_dev(a, dev="cuda"):
    """numpy -> device tensor; uint16 arrays are bf16 bits."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_f64(t):
    """device / host tensor -> fp64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    """max|got - ref| / RMS(ref), RMS over the whole reference tensor."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.abs(got).max(initial=0.0))
    return float(np.abs(got - ref).max(initial=0.0)) / rms


def scaled_excess(got, ref, dtype):
    """Largest per-row  max(|got - ref| - slack) / RMS(ref row).

    Rows are tokens (out), expert rows (a, y) or whatever the last axis
    indexes; a 1-D array is one row.  For bf16 outputs the slack is one bf16
    ulp of the element's own value (2^-8 |ref|), the cost of storing it in
    bf16; fp32 outputs get no slack.  Rows whose reference is all zero must
    be exactly zero (they report inf otherwise).
    """
    got = np.atleast_2d(np.asarray(got, dtype=np.float64))
    ref = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    slack = 2.0 ** -8 * np.abs(ref) if dtype == "bf16" else 0.0
    excess = np.maximum(np.abs(got - ref) - slack, 0.0).max(axis=1)
    rms = np.sqrt(np.mean(ref * ref, axis=1))
    zero = rms == 0.0
    out = np.zeros_like(rms)
    out[~zero] = excess[~zero] / rms[~zero]
    out[zero & (np.abs(got).max(axis=1) > 0)] = np.inf
    return float(out.max(initial=0.0))


def assert_close(got, ref, dtype, what):
    """Parity rule for floats: every row within tau * RMS(that row of ref)
    beyond its storage rounding (see scaled_excess).  Returns the plain
    whole-tensor max|got - ref| / RMS(ref) for reporting."""
    e = scaled_excess(got, ref, dtype)
    assert e <= TAU[dtype], f"{what}: max row excess = {e:.3e} * RMS(row) > {TAU[dtype]}"
    return rel_err(got, ref)


def device_inputs(wl, inp, dev="cuda"):
    d = {k: to_dev(v, dev) for k, v in inp.items()}
    return d


def print_case(*args):
    print("[case]", *args, flush=True)
