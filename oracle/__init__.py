"""CPU oracle for the MoE expert-layer path (fp64).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the GPU library and its
binding never do, and nothing here imports them.

The arithmetic lives in ``moe_oracle.cpp`` (plain fp64 loops, compiled with
g++ -O2 -fopenmp); this module marshals numpy arrays and strings the steps
together in the order the method takes them:

  router logits -> softmax / top-k / renormalise -> stable permute (counts,
  offsets, row_src, inv) -> gather rows -> per-expert SwiGLU FFN with the
  routing scale -> combine back to token order,

and, for the MXFP8 training step, MX quantisation of every GEMM operand along
that GEMM's reduction axis, the forward on the dequantised values, and the
backward by the chain rule.  Passages followed are cited in the C++ source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmoe_oracle.so")

DT_F32, DT_BF16, DT_F64 = 0, 1, 2


def build(force: bool = True) -> str:
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(
            ["g++", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c++17",
             "-o", tmp, os.path.join(_HERE, "moe_oracle.cpp")])
        os.replace(tmp, _SO)
    return _SO


_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(_SO):
            build(force=False)
        L = ctypes.CDLL(_SO)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_router_logits.argtypes = [vp, vp, i32, vp, i64, i64, i64, vp]
        L.orc_topk_softmax.argtypes = [vp, i64, i64, i64, vp, vp]
        L.orc_permute.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, vp]
        L.orc_gather_rows.argtypes = [vp, i32, i64, i64, vp, i64, vp]
        L.orc_expert_ffn_rows.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32,
                                          i64, i64, i64, vp, vp]
        L.orc_combine.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        L.orc_moe_tokens.argtypes = [vp, i32, vp, vp, i64, vp, i64, i64, i64,
                                     vp, vp, vp, i32, i64, i64, vp]
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode_array.argtypes = [vp, i64, vp]
        L.orc_mx_scale_byte.argtypes = [ctypes.c_double]
        L.orc_mx_scale_byte.restype = ctypes.c_uint8
        L.orc_mx_quantize_rows.argtypes = [vp, i64, i64, vp, vp]
        L.orc_mx_dequantize_rows.argtypes = [vp, vp, i64, i64, vp]
        L.orc_e5m2_value.argtypes = [ctypes.c_uint8]
        L.orc_e5m2_value.restype = ctypes.c_double
        L.orc_e5m2_encode.argtypes = [ctypes.c_double]
        L.orc_e5m2_encode.restype = ctypes.c_uint8
        L.orc_e5m2_encode_array.argtypes = [vp, i64, vp]
        L.orc_mx_scale_byte_fmt.argtypes = [ctypes.c_double, ctypes.c_int]
        L.orc_mx_scale_byte_fmt.restype = ctypes.c_uint8
        L.orc_mx_quantize_rows_fmt.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp]
        L.orc_mx_dequantize_rows_fmt.argtypes = [vp, vp, i64, i64, ctypes.c_int, vp]
        L.orc_matmul_nt.argtypes = [vp, vp, i64, i64, i64, vp]
        L.orc_round_bf16.argtypes = [vp, i64, vp]
        L.orc_swiglu_bwd_rows.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp,
                                          vp]
        L.orc_swiglu_rows.argtypes = [vp, vp, vp, i64, i64, vp]
        L.orc_eplb_plan.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp]
        L.orc_permute_replicated.argtypes = [vp, i64, i64, i64, vp, vp, i64,
                                             i64, vp, vp, vp, vp]
        _L = L
    return _L


def _c(a, dtype=None):
    a = np.asarray(a) if dtype is None else np.asarray(a, dtype=dtype)
    return np.ascontiguousarray(a)


def _p(a):
    return None if a is None else a.ctypes.data


def _dt(a):
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.float64:
        return DT_F64
    raise TypeError(f"unsupported dtype {a.dtype}")


# --------------------------------------------------------------------------
# Forward path steps


def router_logits(x, w_router, bias=None):
    """fp64 logits [T, E] = x . w_router^T + bias."""
    x, w = _c(x), _c(w_router)
    assert _dt(x) == _dt(w)
    T, H = x.shape
    E = w.shape[0]
    out = np.empty((T, E), dtype=np.float64)
    b = None if bias is None else _c(bias, np.float32)
    _lib().orc_router_logits(_p(x), _p(w), _dt(x), _p(b), T, H, E, _p(out))
    return out


def topk_softmax(logits_f32, k):
    """Top-k of softmax(logits) renormalised; logits are fp32 [T, E]."""
    l = _c(logits_f32, np.float32)
    T, E = l.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    _lib().orc_topk_softmax(_p(l), T, E, k, _p(idx), _p(w))
    return idx, w


def permute(idx, e_begin, n_local):
    """Stable counting sort of the flat slots by local expert."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(n_local, dtype=np.int32)
    offsets = np.empty(n_local + 1, dtype=np.int32)
    row_src = np.empty(T * k, dtype=np.int32)
    inv = np.empty((T, k), dtype=np.int32)
    _lib().orc_permute(_p(idx), T, k, e_begin, n_local, _p(counts),
                       _p(offsets), _p(row_src), _p(inv))
    R = int(offsets[-1])
    return dict(counts=counts, offsets=offsets, row_src=row_src[:R].copy(),
                inv=inv, R=R)


def gather_rows(x, row_src, k):
    x = _c(x)
    row_src = _c(row_src, np.int32)
    R = row_src.shape[0]
    out = np.empty((R, x.shape[1]), dtype=x.dtype)
    _lib().orc_gather_rows(_p(x), _dt(x), x.shape[1], k, _p(row_src), R,
                           _p(out))
    return out


def expert_ffn_rows(xs, experts, scales, w_gate, w_up, w_down,
                    want_a=True, want_y=True):
    """a = s*SiLU(W_g x)*(W_u x) and y = W_d a for listed rows (fp64)."""
    xs = _c(xs)
    ex = _c(experts, np.int32)
    sc = None if scales is None else _c(scales, np.float64)
    wg, wu, wd = _c(w_gate), _c(w_up), _c(w_down)
    n, H = xs.shape
    I = wg.shape[1]
    a = np.empty((n, I), dtype=np.float64) if want_a else None
    y = np.empty((n, H), dtype=np.float64) if want_y else None
    _lib().orc_expert_ffn_rows(_p(xs), _dt(xs), _p(ex), _p(sc), _p(wg),
                               _p(wu), _p(wd), _dt(wg), n, H, I, _p(a), _p(y))
    return a, y


def combine(y, inv, w=None):
    y = _c(y, np.float64)
    inv = _c(inv, np.int32)
    T, k = inv.shape
    H = y.shape[1]
    out = np.empty((T, H), dtype=np.float64)
    wc = None if w is None else _c(w, np.float64)
    _lib().orc_combine(_p(y), _p(inv), _p(wc), T, k, H, _p(out))
    return out


def moe_tokens(x, idx, w, tokens, e_begin, n_local, w_gate, w_up, w_down):
    """The layer by its definition (no permutation) for listed tokens."""
    x = _c(x)
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    tok = _c(tokens, np.int32)
    wg, wu, wd = _c(w_gate), _c(w_up), _c(w_down)
    H = x.shape[1]
    I = wg.shape[1]
    out = np.empty((tok.shape[0], H), dtype=np.float64)
    _lib().orc_moe_tokens(_p(x), _dt(x), _p(idx), _p(w), idx.shape[1],
                          _p(tok), tok.shape[0], e_begin, n_local, _p(wg),
                          _p(wu), _p(wd), _dt(wg), H, I, _p(out))
    return out


def routing_of(w, inputs):
    """Routing of a workload: (idx, w_topk) from the generated inputs.

    For router == "gemm" the oracle's own fp64 logits are rounded to fp32
    (the precision the GPU path takes its top-k decision in) before top-k.
    Returns (idx, weights, logits_used_fp32, logits_fp64_or_None).
    """
    if "logits" in inputs:
        l32 = np.ascontiguousarray(inputs["logits"], dtype=np.float32)
        l64 = None
    else:
        l64 = router_logits(inputs["x"], inputs["w_router"],
                            inputs.get("bias"))
        l32 = l64.astype(np.float32)
    idx, wts = topk_softmax(l32, w.k)
    return idx, wts, l32, l64


def moe_layer(w, inputs, scale_in_ffn=True):
    """Every step of the forward path on a (small) workload, fp64.

    Returns a dict with logits, idx, topk_w, counts, offsets, row_src, inv,
    x_perm, s_perm, a, y, out.
    """
    idx, wts, l32, l64 = routing_of(w, inputs)
    x = inputs["x"]
    p = permute(idx, w.e_begin, w.n_local)
    R = p["R"]
    x_perm = gather_rows(x, p["row_src"], w.k)
    s_perm = wts.reshape(-1)[p["row_src"]]
    ex = np.repeat(np.arange(w.n_local, dtype=np.int32), p["counts"])
    a, y = expert_ffn_rows(x_perm, ex, s_perm if scale_in_ffn else None,
                           inputs["w_gate"], inputs["w_up"], inputs["w_down"])
    out = combine(y, p["inv"], None if scale_in_ffn else wts)
    return dict(logits=l64 if l64 is not None else l32, idx=idx, topk_w=wts,
                counts=p["counts"], offsets=p["offsets"],
                row_src=p["row_src"], inv=p["inv"], R=R, x_perm=x_perm,
                s_perm=s_perm, a=a, y=y, out=out)


# --------------------------------------------------------------------------
# Expert-parallel load balancing


def eplb_plan(counts, n_slots, n_ranks):
    """Replicas and placement of E experts with observed `counts` on n_slots
    physical slots over n_ranks ranks (see orc_eplb_plan).  Returns dict rep
    [E], rep_first [E+1], rep_slot [S], slot_expert [S], slot_copy [S]."""
    c = _c(counts, np.int32)
    E = c.shape[0]
    S = int(n_slots)
    out = dict(rep=np.empty(E, np.int32), rep_first=np.empty(E + 1, np.int32),
               rep_slot=np.empty(S, np.int32), slot_expert=np.empty(S, np.int32),
               slot_copy=np.empty(S, np.int32))
    _lib().orc_eplb_plan(_p(c), E, S, int(n_ranks), _p(out["rep"]),
                         _p(out["rep_first"]), _p(out["rep_slot"]),
                         _p(out["slot_expert"]), _p(out["slot_copy"]))
    return out


def permute_replicated(idx, E, plan, s_begin, n_slots):
    """Stable dispatch of the flat entries to the slots [s_begin, s_begin +
    n_slots) of a plan, splitting each expert's current entries among its
    copies (see orc_permute_replicated)."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(n_slots, np.int32)
    offsets = np.empty(n_slots + 1, np.int32)
    row_src = np.empty(T * k, np.int32)
    inv = np.empty((T, k), np.int32)
    _lib().orc_permute_replicated(
        _p(idx), T, k, int(E), _p(_c(plan["rep_first"], np.int32)),
        _p(_c(plan["rep_slot"], np.int32)), int(s_begin), int(n_slots),
        _p(counts), _p(offsets), _p(row_src), _p(inv))
    R = int(offsets[-1])
    return dict(counts=counts, offsets=offsets, row_src=row_src[:R].copy(),
                inv=inv, R=R)


def copy_rows(n, r, i):
    """Rows [lo, hi) of copy i among r copies of an expert with n rows."""
    return i * n // r, (i + 1) * n // r


# --------------------------------------------------------------------------
# MXFP8


def e4m3_value(code):
    return _lib().orc_e4m3_value(int(code))


def e4m3_encode(v):
    return int(_lib().orc_e4m3_encode(float(v)))


def e4m3_encode_array(v):
    """E4M3 codes (nearest, ties to even, saturating) of every value."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    _lib().orc_e4m3_encode_array(_p(v), v.size, _p(out))
    return out


# Element formats of MX blocks: E4M3 (the default for every operand) and
# E5M2 (the gradient option).
MX_FORMATS = {"e4m3": 0, "e5m2": 1}


def _fmt(fmt):
    try:
        return MX_FORMATS[fmt]
    except KeyError:
        raise ValueError(f"unknown MX element format {fmt!r}") from None


def e5m2_value(code):
    return _lib().orc_e5m2_value(int(code))


def e5m2_encode(v):
    return int(_lib().orc_e5m2_encode(float(v)))


def e5m2_encode_array(v):
    """E5M2 codes (nearest, ties to even, saturating) of every value."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    _lib().orc_e5m2_encode_array(_p(v), v.size, _p(out))
    return out


def mx_scale_byte(amax, fmt="e4m3"):
    return int(_lib().orc_mx_scale_byte_fmt(float(amax), _fmt(fmt)))


def mx_quantize_rows(v, fmt="e4m3"):
    """Blocks of 32 along each row: (codes [r, c] u8, scales [r, ceil(c/32)]),
    elements of format fmt."""
    v = _c(v, np.float64)
    r, c = v.shape
    codes = np.empty((r, c), dtype=np.uint8)
    scales = np.empty((r, (c + 31) // 32), dtype=np.uint8)
    _lib().orc_mx_quantize_rows_fmt(_p(v), r, c, _fmt(fmt), _p(codes), _p(scales))
    return codes, scales


def mx_dequantize_rows(codes, scales, fmt="e4m3"):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    r, c = codes.shape
    v = np.empty((r, c), dtype=np.float64)
    _lib().orc_mx_dequantize_rows_fmt(_p(codes), _p(scales), r, c, _fmt(fmt), _p(v))
    return v


def mx_roundtrip_rows(v, fmt="e4m3"):
    """Dequantised MX values of v, blocks of 32 along each row."""
    return mx_dequantize_rows(*mx_quantize_rows(v, fmt), fmt=fmt)


def mx_roundtrip_cols(v, fmt="e4m3"):
    """Dequantised MX values of v, blocks of 32 down each column."""
    return np.ascontiguousarray(mx_roundtrip_rows(np.ascontiguousarray(v.T), fmt).T)


def to_f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_bf16(v):
    """Nearest bfloat16 value of each element (ties to even), as fp64."""
    v = _c(v, np.float64)
    out = np.empty_like(v)
    _lib().orc_round_bf16(_p(v), v.size, _p(out))
    return out


def matmul_nt(A, B):
    A, B = _c(A, np.float64), _c(B, np.float64)
    M, K = A.shape
    N = B.shape[0]
    C = np.empty((M, N), dtype=np.float64)
    _lib().orc_matmul_nt(_p(A), _p(B), M, N, K, _p(C))
    return C


def swiglu_bwd(da, g, u, s):
    da, g, u, s = (_c(t, np.float64) for t in (da, g, u, s))
    R, I = da.shape
    dg = np.empty((R, I)); du = np.empty((R, I)); ds = np.empty(R)
    _lib().orc_swiglu_bwd_rows(_p(da), _p(g), _p(u), _p(s), R, I, _p(dg),
                               _p(du), _p(ds))
    return dg, du, ds


def swiglu(g, u, s=None):
    """a = s * SiLU(g) * u (ScaledSwiGLU) of given pre-activations, fp64."""
    g, u = _c(g, np.float64), _c(u, np.float64)
    R, I = g.shape
    sc = None if s is None else _c(s, np.float64)
    a = np.empty((R, I))
    _lib().orc_swiglu_rows(_p(g), _p(u), _p(sc), R, I, _p(a))
    return a


def mx_gemm_nt(A, B, quantize=True, fmt_a="e4m3", fmt_b="e4m3"):
    """C = Q(A) . Q(B)^T with every row of A [M, K] and of B [N, K]
    MX-quantised along K (blocks of 32 from column 0; a shorter last block is
    a block padded with zeros) and the dequantised values multiplied exactly
    in fp64.  This is the one MXFP8 GEMM of the step: every operand is
    blocked along its GEMM's reduction axis [TE-MXFP8], which a caller
    chooses by the orientation it passes.  fmt_a, fmt_b: element formats of
    the two operands.  quantize=False: plain product."""
    A, B = _c(A, np.float64), _c(B, np.float64)
    if quantize:
        A, B = mx_roundtrip_rows(A, fmt_a), mx_roundtrip_rows(B, fmt_b)
    return matmul_nt(A, B)


def _T(v):
    return np.ascontiguousarray(np.asarray(v, dtype=np.float64).T)


def mxfp8_forward(x_perm, offsets, s_perm, w_gate, w_up, w_down,
                  quantize=True):
    """MXFP8 grouped MLP forward on permuted rows [TE-Grouped, TE-MXFP8]:
    per expert e and its rows, g = Q_H(x) Q_H(W_g)^T, u likewise,
    a = s SiLU(g) u (fp64, not rounded), y = Q_I(a) Q_I(W_d)^T.
    Inputs bf16 bits (uint16) or fp64; returns dict of fp64 g, u, a, y."""
    x = to_f64(x_perm)
    s = np.asarray(s_perm, dtype=np.float64)
    n_local = len(offsets) - 1
    R, H = x.shape
    I = w_gate.shape[1]
    g = np.zeros((R, I)); u = np.zeros((R, I)); a = np.zeros((R, I))
    y = np.zeros((R, H))
    for e in range(n_local):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        xe = x[r0:r1]
        g[r0:r1] = mx_gemm_nt(xe, to_f64(w_gate[e]), quantize)
        u[r0:r1] = mx_gemm_nt(xe, to_f64(w_up[e]), quantize)
        a[r0:r1] = swiglu(g[r0:r1], u[r0:r1], s[r0:r1])
        y[r0:r1] = mx_gemm_nt(a[r0:r1], to_f64(w_down[e]), quantize)
    return dict(g=g, u=u, a=a, y=y)


def mxfp8_wgrad(A, B, offsets, quantize=True, fmt_a="e4m3"):
    """Weight gradient per expert: W[e] = Q_R(A_e)^T Q_R(B_e) over expert
    e's rows (A [R, M], B [R, N] -> [n_local, M, N]), every operand blocked
    down the rows of the segment from its first row (the GEMM's reduction
    axis); an expert without rows gets zeros.  A is the gradient operand
    (elements of format fmt_a), B an activation (E4M3)."""
    A, B = to_f64(A), to_f64(B)
    n_local = len(offsets) - 1
    out = np.zeros((n_local, A.shape[1], B.shape[1]))
    for e in range(n_local):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            out[e] = mx_gemm_nt(_T(A[r0:r1]), _T(B[r0:r1]), quantize, fmt_a)
    return out


def mxfp8_backward_down(dy, g, u, s_perm, offsets, w_down, quantize=True,
                        grad_fmt="e4m3"):
    """Backward of the down projection and of ScaledSwiGLU, by the chain
    rule: da = Q_H(dY) Q_H(W_d) per expert (K = H), dg, du, ds from
    swiglu_bwd at the given g, u, and dW_d = Q_R(dY)^T Q_R(a) with a =
    s SiLU(g) u.  grad_fmt: element format of the gradient operand dY (W_d
    and a stay E4M3).  Returns dict of fp64 da, dg, du, ds, a, dw_down."""
    dY = to_f64(dy)
    g, u = to_f64(g), to_f64(u)
    s = np.asarray(s_perm, dtype=np.float64)
    n_local = len(offsets) - 1
    R, I = g.shape
    da = np.zeros((R, I)); dg = np.zeros((R, I)); du = np.zeros((R, I))
    ds = np.zeros(R)
    for e in range(n_local):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        # W_d[e] is [H, I]; da[r, i] = sum_h dY[r, h] W_d[h, i]
        da[r0:r1] = mx_gemm_nt(dY[r0:r1], _T(to_f64(w_down[e])), quantize,
                               grad_fmt)
        dg[r0:r1], du[r0:r1], ds[r0:r1] = swiglu_bwd(
            da[r0:r1], g[r0:r1], u[r0:r1], s[r0:r1])
    a = swiglu(g, u, s)
    dwd = mxfp8_wgrad(dY, a, offsets, quantize, grad_fmt)
    return dict(da=da, dg=dg, du=du, ds=ds, a=a, dw_down=dwd)


def mxfp8_backward_gate_up(dg, du, x_perm, offsets, w_gate, w_up,
                           quantize=True, grad_fmt="e4m3"):
    """Backward of the gate/up projection: dX = Q_I(dg) Q_I(W_g) +
    Q_I(du) Q_I(W_u) per expert (K = I), dW_g = Q_R(dg)^T Q_R(x),
    dW_u = Q_R(du)^T Q_R(x).  grad_fmt: element format of the gradient
    operands dg, du (W_g, W_u and x stay E4M3).  Returns dict of fp64 dx,
    dw_gate, dw_up."""
    dg, du, x = to_f64(dg), to_f64(du), to_f64(x_perm)
    n_local = len(offsets) - 1
    R, H = x.shape
    dx = np.zeros((R, H))
    for e in range(n_local):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        # W_g[e] is [I, H]; dX[r, h] = sum_i dg[r, i] W_g[i, h] + du W_u
        dx[r0:r1] = (mx_gemm_nt(dg[r0:r1], _T(to_f64(w_gate[e])), quantize,
                                grad_fmt)
                     + mx_gemm_nt(du[r0:r1], _T(to_f64(w_up[e])), quantize,
                                  grad_fmt))
    return dict(dx=dx, dw_gate=mxfp8_wgrad(dg, x, offsets, quantize, grad_fmt),
                dw_up=mxfp8_wgrad(du, x, offsets, quantize, grad_fmt))


def mxfp8_mlp_step(x_perm, offsets, s_perm, w_gate, w_up, w_down, dy,
                   quantize=True, bf16_dgu=False, grad_fmt="e4m3"):
    """MXFP8 grouped MLP forward + backward on permuted rows, fp64: the
    forward, the down/SwiGLU backward at the forward's own g, u, and the
    gate/up backward.  Every GEMM operand is MX-quantised along that GEMM's
    reduction axis (mx_gemm_nt); no tensor is rounded to bf16 on the way
    (the quantisation is fused with SwiGLU and the scaling [TE-MXFP8]).
    quantize=False: the same chain rule on unquantised operands (what the
    finite-difference pins check).  bf16_dgu=True: dg and du are rounded to
    bf16 before the gate/up backward quantises them, as the unfused stage
    API hands [dg | du] from one call to the next in bf16 (a labelled
    variant for that API only).  grad_fmt: element format of every gradient
    operand (dY, dg, du) of the backward GEMMs, "e4m3" or "e5m2"; weights and
    activations stay E4M3.  Returns fp64 g, u, a, y, da, dg, du, ds, dx,
    dw_gate, dw_up, dw_down."""
    f = mxfp8_forward(x_perm, offsets, s_perm, w_gate, w_up, w_down, quantize)
    b = mxfp8_backward_down(dy, f["g"], f["u"], s_perm, offsets, w_down,
                            quantize, grad_fmt)
    dg, du = b["dg"], b["du"]
    if bf16_dgu:
        dg, du = round_bf16(dg), round_bf16(du)
    c = mxfp8_backward_gate_up(dg, du, x_perm, offsets, w_gate, w_up,
                               quantize, grad_fmt)
    return dict(g=f["g"], u=f["u"], a=f["a"], y=f["y"], da=b["da"],
                dg=b["dg"], du=b["du"], ds=b["ds"], dx=c["dx"],
                dw_gate=c["dw_gate"], dw_up=c["dw_up"],
                dw_down=b["dw_down"])
