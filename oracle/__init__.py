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
        L.orc_gate_up_rows.argtypes = [vp, i32, vp, vp, vp, i32, i64, i64,
                                       i64, vp, vp]
        L.orc_combine.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        L.orc_moe_tokens.argtypes = [vp, i32, vp, vp, i64, vp, i64, i64, i64,
                                     vp, vp, vp, i32, i64, i64, vp]
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_mx_scale_byte.argtypes = [ctypes.c_double]
        L.orc_mx_scale_byte.restype = ctypes.c_uint8
        L.orc_mx_quantize_rows.argtypes = [vp, i64, i64, vp, vp]
        L.orc_mx_dequantize_rows.argtypes = [vp, vp, i64, i64, vp]
        L.orc_matmul_nt.argtypes = [vp, vp, i64, i64, i64, vp]
        L.orc_round_bf16.argtypes = [vp, i64, vp]
        L.orc_swiglu_bwd_rows.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp,
                                          vp]
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


def gate_up_rows(xs, experts, w_gate, w_up):
    xs = _c(xs)
    ex = _c(experts, np.int32)
    wg, wu = _c(w_gate), _c(w_up)
    n, H = xs.shape
    I = wg.shape[1]
    g = np.empty((n, I), dtype=np.float64)
    u = np.empty((n, I), dtype=np.float64)
    _lib().orc_gate_up_rows(_p(xs), _dt(xs), _p(ex), _p(wg), _p(wu), _dt(wg),
                            n, H, I, _p(g), _p(u))
    return g, u


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
# MXFP8


def e4m3_value(code):
    return _lib().orc_e4m3_value(int(code))


def e4m3_encode(v):
    return int(_lib().orc_e4m3_encode(float(v)))


def mx_scale_byte(amax):
    return int(_lib().orc_mx_scale_byte(float(amax)))


def mx_quantize_rows(v):
    """Blocks of 32 along each row: (codes [r, c] u8, scales [r, ceil(c/32)])."""
    v = _c(v, np.float64)
    r, c = v.shape
    codes = np.empty((r, c), dtype=np.uint8)
    scales = np.empty((r, (c + 31) // 32), dtype=np.uint8)
    _lib().orc_mx_quantize_rows(_p(v), r, c, _p(codes), _p(scales))
    return codes, scales


def mx_dequantize_rows(codes, scales):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    r, c = codes.shape
    v = np.empty((r, c), dtype=np.float64)
    _lib().orc_mx_dequantize_rows(_p(codes), _p(scales), r, c, _p(v))
    return v


def mx_roundtrip_rows(v):
    """Dequantised MX values of v, blocks of 32 along each row."""
    return mx_dequantize_rows(*mx_quantize_rows(v))


def mx_roundtrip_cols(v):
    """Dequantised MX values of v, blocks of 32 down each column."""
    return np.ascontiguousarray(mx_roundtrip_rows(np.ascontiguousarray(v.T)).T)


def mx_roundtrip_cols_segmented(v, offsets):
    """Blocks of 32 down each column, restarting at every segment start."""
    out = np.empty(v.shape, dtype=np.float64)
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            out[a:b] = mx_roundtrip_cols(v[a:b])
    return out


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


def mxfp8_mlp_step(x_perm, offsets, s_perm, w_gate, w_up, w_down, dy,
                   quantize=True, handoff=None):
    """MXFP8 grouped MLP forward + backward on permuted rows, fp64.

    Every GEMM operand is MX-quantised (blocks of 32) along that GEMM's
    reduction axis; products of the dequantised values are exact in fp64.
      forward:  g = Q_H(x) Q_H(W_g)^T, u likewise, a = s*SiLU(g)*u,
                y = Q_I(a) Q_I(W_d)^T
      backward: da = Q_H(dY) Q_H(W_d), dg/du/ds by the chain rule,
                dX = Q_I(dg) Q_I(W_g) + Q_I(du) Q_I(W_u),
                dW_d[e] = Q_R(dY_e)^T Q_R(a_e), dW_g[e] = Q_R(dg_e)^T Q_R(x_e),
                dW_u[e] = Q_R(du_e)^T Q_R(x_e)
    with Q_R blocking along the rows of each expert's segment.
    All inputs are bf16 bits (uint16) or fp64; returns fp64 arrays.
    ``quantize=False`` replaces every Q by the identity (the same chain rule
    on unquantised operands), which the finite-difference pins check.

    ``handoff`` (default: same as ``quantize``) stores the tensors that pass
    from one operation to the next in bf16 before they are used, as in a
    BF16 training step whose GEMMs run in MXFP8 ([TE-MXFP8]): a before the
    down projection and its weight gradient, the saved g and u before the
    SwiGLU backward, dg and du before their GEMMs.  Each quantisation then
    starts from the bf16 tensor, as it does on the device.  The returned
    g, u, a, dg, du are the fp64 values before that rounding.
    """
    if handoff is None:
        handoff = quantize
    bf = round_bf16 if handoff else (lambda v: v)
    if quantize:
        q_rows, q_cols = mx_roundtrip_rows, mx_roundtrip_cols
    else:
        q_rows = q_cols = (lambda v: np.array(v, dtype=np.float64))
    x = to_f64(x_perm)
    dY = to_f64(dy)
    s = np.asarray(s_perm, dtype=np.float64)
    n_local = len(offsets) - 1
    R, H = x.shape
    I = w_gate.shape[1]
    xq = q_rows(x)
    dyq_h = q_rows(dY)
    g = np.zeros((R, I)); u = np.zeros((R, I)); a = np.zeros((R, I))
    y = np.zeros((R, H)); da = np.zeros((R, I))
    dx = np.zeros((R, H)); ds = np.zeros(R)
    dwg = np.zeros((n_local, I, H)); dwu = np.zeros((n_local, I, H))
    dwd = np.zeros((n_local, H, I))
    dg = np.zeros((R, I)); du = np.zeros((R, I))
    for e in range(n_local):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        Wg, Wu, Wd = (to_f64(t[e]) for t in (w_gate, w_up, w_down))
        if r1 == r0:
            continue
        xe = xq[r0:r1]
        g[r0:r1] = matmul_nt(xe, q_rows(Wg))
        u[r0:r1] = matmul_nt(xe, q_rows(Wu))
        a[r0:r1] = s[r0:r1, None] * (g[r0:r1] / (1.0 + np.exp(-g[r0:r1]))) * u[r0:r1]
        a_h = bf(a[r0:r1])
        y[r0:r1] = matmul_nt(q_rows(a_h), q_rows(Wd))
        # dgrad of down: da[r, i] = sum_h dY[r, h] Wd[h, i], K = H
        da[r0:r1] = matmul_nt(dyq_h[r0:r1], np.ascontiguousarray(q_cols(Wd).T))
        dg[r0:r1], du[r0:r1], ds[r0:r1] = swiglu_bwd(
            da[r0:r1], bf(g[r0:r1]), bf(u[r0:r1]), s[r0:r1])
        dg_h, du_h = bf(dg[r0:r1]), bf(du[r0:r1])
        # dgrad of gate/up: dX[r, h] = sum_i dg[r,i] Wg[i,h] + du[r,i] Wu[i,h]
        WgT = np.ascontiguousarray(q_cols(Wg).T)
        WuT = np.ascontiguousarray(q_cols(Wu).T)
        dx[r0:r1] = (matmul_nt(q_rows(dg_h), WgT)
                     + matmul_nt(q_rows(du_h), WuT))
        # wgrad: reduction over the segment's rows
        dyr = np.ascontiguousarray(q_cols(dY[r0:r1]).T)   # [H, n]
        ar = np.ascontiguousarray(q_cols(a_h).T)          # [I, n]
        xr = np.ascontiguousarray(q_cols(x[r0:r1]).T)     # [H, n]
        dgr = np.ascontiguousarray(q_cols(dg_h).T)        # [I, n]
        dur = np.ascontiguousarray(q_cols(du_h).T)
        dwd[e] = matmul_nt(dyr, ar)
        dwg[e] = matmul_nt(dgr, xr)
        dwu[e] = matmul_nt(dur, xr)
    return dict(g=g, u=u, a=a, y=y, da=da, dg=dg, du=du, ds=ds, dx=dx,
                dw_gate=dwg, dw_up=dwu, dw_down=dwd)
