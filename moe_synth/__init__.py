"""Seeded synthetic inputs for the MoE expert-layer path.

This module draws inputs only: token activations, router and expert weights,
the per-expert Zipf logit bias, generated router logits and upstream
gradients.  It holds none of the method's arithmetic (no routing, no
permutation of tokens, no expert FFN), so both the CPU oracle and the GPU path
may read it.  The generator itself is defined in ``synth.c`` (SplitMix64 in
counter mode, Box-Muller in fp64, round-to-nearest-even to the storage dtype).

Workload presets follow the shapes the pages give for DeepSeek-R1 (256 experts
per layer, 8 routed per token; NVIDIA Wide-EP explainer, "Premise: what MoE
is") and its EP64 / EP8 expert shares (4 and 32 experts per GPU; same page,
"Wide-EP" section, and the SemiAnalysis WideEP excerpt, "Context Before"), plus
an E=8/top-2 MXFP8 MLP like the BioNeMo recipe's Mixtral-shaped run (BioNeMo
article, "BioNeMo Recipe Achieves 2.21x").
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmoe_synth.so")

# Stream ids: one independent counter stream per tensor.
STREAM_X = 1
STREAM_W_ROUTER = 2
STREAM_ZIPF_PERM = 3
STREAM_LOGITS = 4
STREAM_W_GATE = 10
STREAM_W_UP = 11
STREAM_W_DOWN = 12
STREAM_DY = 20
STREAM_A = 21
STREAM_GU = 22
STREAM_DGU = 23


def build(force: bool = True) -> str:
    """Compile the generator with gcc (OpenMP) into ``libmoe_synth.so``."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp,
             os.path.join(_HERE, "synth.c"), "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_SO):
            build(force=False)
        L = ctypes.CDLL(_SO)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.c_double,
                                  ctypes.c_void_p)
        L.synth_normal_f32.argtypes = [u64, u64, u64, u64, dbl, dbl, vp]
        L.synth_normal_bf16.argtypes = [u64, u64, u64, u64, dbl, dbl, vp]
        L.synth_permutation.argtypes = [u64, u64, i32, vp]
        L.synth_zipf_bias.argtypes = [u64, u64, i32, dbl, vp]
        L.synth_biased_logits.argtypes = [u64, u64, i64, i32, vp, vp]
        L.synth_stream_key.argtypes = [u64, u64]
        L.synth_stream_key.restype = u64
        _lib_handle = L
    return _lib_handle


def _ptr(a) -> int:
    if isinstance(a, np.ndarray):
        assert a.flags["C_CONTIGUOUS"]
        return a.ctypes.data
    return int(a)


def normal_f32(seed, stream, offset, n, mean, std, out=None):
    """fp32 normal deviates of elements [offset, offset+n) of a stream."""
    if out is None:
        out = np.empty(n, dtype=np.float32)
    _lib().synth_normal_f32(seed, stream, offset, n, mean, std, _ptr(out))
    return out


def normal_bf16(seed, stream, offset, n, mean, std, out=None):
    """bf16 (raw uint16 bits) normal deviates of elements [offset, offset+n)."""
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    _lib().synth_normal_bf16(seed, stream, offset, n, mean, std, _ptr(out))
    return out


def permutation(seed, stream, n):
    out = np.empty(n, dtype=np.int32)
    _lib().synth_permutation(seed, stream, n, _ptr(out))
    return out


def zipf_bias(seed, n_experts, s):
    """Zipf bias: a seeded shuffle orders the experts by popularity; the one
    at position i gets b = (1 + i)^(-s)."""
    out = np.empty(n_experts, dtype=np.float64)
    _lib().synth_zipf_bias(seed, STREAM_ZIPF_PERM, n_experts, s, _ptr(out))
    return out


def biased_logits(seed, T, E, bias=None):
    """fp32 logits[t, e] = N(0,1) + bias[e] (bias in fp64, or none)."""
    out = np.empty((T, E), dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
    _lib().synth_biased_logits(seed, STREAM_LOGITS, T, E,
                               None if b is None else _ptr(b), _ptr(out))
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to fp32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One seeded synthetic workload.

    router: "gemm"   -> logits = x . W_r^T (+ bias), routing computed on the path
            "logits" -> logits are drawn directly (N(0,1) + bias); routing of
                        these logits happens before the timed path
    Weights are stored K-contiguous: W_r [E, H], W_gate/W_up [E, I, H],
    W_down [E, H, I].  Experts [e_begin, e_begin + n_local) are this GPU's.
    """
    name: str
    dtype: str          # "f32", "bf16" or "mxfp8"
    T: int              # tokens on the path
    H: int              # hidden size
    I: int              # intermediate size per expert
    E: int              # experts the router chooses among
    k: int              # experts per token
    e_begin: int
    n_local: int
    router: str
    zipf_s: float | None
    w_std: float = 0.02
    seed: int = 0

    @property
    def act_dtype(self) -> str:
        return "f32" if self.dtype == "f32" else "bf16"


WORKLOADS = {
    # Tiny fp32 layer: full path including the router GEMM.
    "c1_tiny_f32": Workload("c1_tiny_f32", "f32", 64, 256, 512, 8, 2, 0, 8,
                            "gemm", None),
    # EP64 share of a DeepSeek-R1-shaped layer: 4096 tokens routed top-8 of
    # 256 with Gaussian + Zipf(1.1) logits, experts 0-3 kept.
    "c2_ep64_bf16": Workload("c2_ep64_bf16", "bf16", 4096, 7168, 2048, 256, 8,
                             0, 4, "logits", 1.1),
    # EP8 share: tokens 0-511 of the same routing, experts 0-31 kept.
    "c3_ep8_bf16": Workload("c3_ep8_bf16", "bf16", 512, 7168, 2048, 256, 8,
                            0, 32, "logits", 1.1),
    # EP8 share read literally: all 4096 tokens of the same routing, experts
    # 0-31 kept (about 128 rows per expert).
    "c3_literal_ep8_bf16": Workload("c3_literal_ep8_bf16", "bf16", 4096, 7168,
                                    2048, 256, 8, 0, 32, "logits", 1.1),
    # Full layer on one GPU: router GEMM + Zipf(1.2) bias, all 256 experts.
    "c4_full_bf16": Workload("c4_full_bf16", "bf16", 8192, 7168, 2048, 256, 8,
                             0, 256, "gemm", 1.2),
    # MXFP8 grouped MLP training step, uniform Gaussian routing top-2 of 8.
    "c5_mxfp8": Workload("c5_mxfp8", "mxfp8", 16384, 4096, 8192, 8, 2, 0, 8,
                         "logits", None),
    # The bf16 forward on the MXFP8 step's shapes (about 4096 rows per
    # expert): a compute-bound grouped FFN.
    "c5_shape_bf16": Workload("c5_shape_bf16", "bf16", 16384, 4096, 8192, 8, 2,
                              0, 8, "logits", None),
    # Small presets for tests (several tiles plus ragged tails).
    "tiny_f32": Workload("tiny_f32", "f32", 16, 64, 128, 4, 2, 0, 4,
                         "gemm", None),
    "tiny_bf16": Workload("tiny_bf16", "bf16", 48, 128, 256, 8, 2, 0, 8,
                          "gemm", 1.2),
    "small_bf16": Workload("small_bf16", "bf16", 300, 512, 384, 16, 4, 0, 16,
                           "gemm", 1.2),
    "small_ep_bf16": Workload("small_ep_bf16", "bf16", 333, 384, 320, 32, 4,
                              8, 8, "logits", 1.1),
    "mid_bf16": Workload("mid_bf16", "bf16", 1024, 1024, 768, 32, 4, 0, 32,
                         "gemm", 1.2),
    "small_mxfp8": Workload("small_mxfp8", "mxfp8", 200, 512, 512, 4, 2, 0, 4,
                            "logits", None),
    "mid_mxfp8": Workload("mid_mxfp8", "mxfp8", 1000, 512, 1024, 8, 2, 0, 8,
                          "logits", None),
}


def _draw(dtype, seed, stream, offset, n, mean, std):
    if dtype == "f32":
        return normal_f32(seed, stream, offset, n, mean, std)
    return normal_bf16(seed, stream, offset, n, mean, std)


def make_inputs(w: Workload, with_weights: bool = True,
                tokens: int | None = None) -> dict:
    """Draw every input of a workload as numpy arrays.

    Floating tensors in bf16 are returned as raw uint16 bits; in fp32 as
    float32.  Keys: x [T,H]; logits [T,E] (router == "logits") or w_router
    [E,H] (+ bias [E] fp32 when zipf_s is set); w_gate, w_up [n_local,I,H];
    w_down [n_local,H,I].  ``tokens`` draws only the first rows of x/logits.
    """
    T = w.T if tokens is None else tokens
    adt = w.act_dtype
    out = {}
    out["x"] = _draw(adt, w.seed, STREAM_X, 0, T * w.H, 0.0, 1.0).reshape(T, w.H)
    bias = zipf_bias(w.seed, w.E, w.zipf_s) if w.zipf_s is not None else None
    if w.router == "logits":
        out["logits"] = biased_logits(w.seed, T, w.E, bias)
    else:
        out["w_router"] = _draw(adt, w.seed, STREAM_W_ROUTER, 0, w.E * w.H,
                                0.0, w.w_std).reshape(w.E, w.H)
        if bias is not None:
            out["bias"] = bias.astype(np.float32)
    if with_weights:
        out.update(make_weights(w))
    return out


def make_weights(w: Workload, experts: range | None = None) -> dict:
    """Expert weights of the local experts (or a sub-range of them)."""
    if experts is None:
        experts = range(w.e_begin, w.e_begin + w.n_local)
    e0, n = experts.start, len(experts)
    wdt = "f32" if w.dtype == "f32" else "bf16"
    IH = w.I * w.H
    return {
        "w_gate": _draw(wdt, w.seed, STREAM_W_GATE, e0 * IH, n * IH, 0.0,
                        w.w_std).reshape(n, w.I, w.H),
        "w_up": _draw(wdt, w.seed, STREAM_W_UP, e0 * IH, n * IH, 0.0,
                      w.w_std).reshape(n, w.I, w.H),
        "w_down": _draw(wdt, w.seed, STREAM_W_DOWN, e0 * IH, n * IH, 0.0,
                        w.w_std).reshape(n, w.H, w.I),
    }


def make_dy(w: Workload, rows: int) -> np.ndarray:
    """Upstream gradient of the expert outputs, [rows, H] bf16 N(0,1)."""
    return normal_bf16(w.seed, STREAM_DY, 0, rows * w.H, 0.0,
                       1.0).reshape(rows, w.H)


def make_handoffs(w: Workload, rows: int) -> dict:
    """Stand-alone bf16 tensors of the shapes the MXFP8 MLP step hands from
    one operation to the next, for testing each GEMM stage on its own:
    a [rows, I] ~ N(0, 0.5), gu = [g | u] [rows, 2I] ~ N(0, 1.25) (the spread
    of x . W for x ~ N(0,1), W ~ N(0, 0.02), H = 4096), dgu = [dg | du]
    [rows, 2I] ~ N(0, 0.5)."""
    I = w.I
    return {
        "a": normal_bf16(w.seed, STREAM_A, 0, rows * I, 0.0, 0.5).reshape(rows, I),
        "gu": normal_bf16(w.seed, STREAM_GU, 0, rows * 2 * I, 0.0,
                          1.25).reshape(rows, 2 * I),
        "dgu": normal_bf16(w.seed, STREAM_DGU, 0, rows * 2 * I, 0.0,
                           0.5).reshape(rows, 2 * I),
    }
