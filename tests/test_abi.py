"""The C-ABI library on the host: it loads, exports every function the header
declares, and rejects bad arguments before anything is enqueued.  None of
these calls reaches a GPU (validation returns first), so they run on CPU."""
import ctypes
import os
import re

import pytest

import mixture_experts_expert_router_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
E_ARG, E_SHAPE, E_ALIGN, E_WS = 1, 2, 3, 4
F32, BF16 = 0, 1
P = 4096        # a fake, 16-byte aligned "device pointer" (never dereferenced)
P_ODD = 4098    # misaligned


@pytest.fixture(scope="module")
def L():
    return moe.lib()


def test_every_declared_symbol_is_exported(L):
    names = moe.declared_functions()
    assert {"moe_route_topk", "moe_permute", "moe_grouped_ffn",
            "moe_unpermute_combine"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    assert moe.status_string(0) == "ok"
    for s in range(1, 7):
        assert moe.status_string(s) not in ("ok", "unknown status")
    assert moe.status_string(99) == "unknown status"
    assert moe.version() >= 100


def test_workspace_queries_are_pure(L):
    a = L.moe_permute_workspace_bytes(8192, 8, 256)
    assert a > 0 and a % 256 == 0
    assert L.moe_permute_workspace_bytes(8192, 8, 256) == a
    assert L.moe_permute_workspace_bytes(-1, 8, 256) == 0
    b = L.moe_grouped_ffn_workspace_bytes(65536, 256, 7168, 2048, BF16)
    assert b >= 257 * 4 and b % 256 == 0
    assert L.moe_grouped_ffn_workspace_bytes(10, 0, 64, 64, BF16) == 0


def test_route_topk_validation(L):
    f = L.moe_route_topk
    # bad dtype, k > E, E too large, k too large
    assert f(None, None, None, P, 4, 0, 8, 2, 7, P, P, None) == E_ARG
    assert f(None, None, None, P, 4, 0, 8, 9, F32, P, P, None) == E_SHAPE
    assert f(None, None, None, P, 4, 0, 2048, 2, F32, P, P, None) == E_SHAPE
    assert f(None, None, None, P, 4, 0, 64, 33, F32, P, P, None) == E_SHAPE
    # x without w_router; bias in logits mode; missing outputs
    assert f(P, None, None, P, 4, 64, 8, 2, BF16, P, P, None) == E_ARG
    assert f(None, None, P, P, 4, 0, 8, 2, F32, P, P, None) == E_ARG
    assert f(None, None, None, None, 4, 0, 8, 2, F32, P, P, None) == E_ARG
    # bf16 router GEMM needs H % 64 == 0 and aligned operands
    assert f(P, P, None, P, 4, 96, 8, 2, BF16, P, P, None) == E_SHAPE
    assert f(P_ODD, P, None, P, 4, 128, 8, 2, BF16, P, P, None) == E_ALIGN
    # nothing to do
    assert f(None, None, None, None, 0, 0, 8, 2, F32, None, None, None) == 0


def test_permute_validation(L):
    f = L.moe_permute
    ws = L.moe_permute_workspace_bytes(16, 2, 4)
    ok = dict(idx=P, w=P, x=P, T=16, k=2, H=64, dt=BF16, E=8, eb=0, nl=4,
              xp=P, sp=P, rs=P, inv=P, cnt=P, off=P, ws=P, wsb=ws)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["idx"], a["w"], a["x"], a["T"], a["k"], a["H"], a["dt"],
                 a["E"], a["eb"], a["nl"], a["xp"], a["sp"], a["rs"],
                 a["inv"], a["cnt"], a["off"], a["ws"], a["wsb"], None)

    assert call(dt=5) == E_ARG
    assert call(k=0) == E_SHAPE and call(k=33) == E_SHAPE
    assert call(nl=0) == E_SHAPE and call(nl=5000) == E_SHAPE
    assert call(eb=-1) == E_SHAPE
    # the local experts must lie inside [0, E)
    assert call(E=0) == E_SHAPE and call(E=3) == E_SHAPE
    assert call(eb=5) == E_SHAPE and call(eb=4) != E_SHAPE
    assert call(E=1 << 31) == E_SHAPE
    assert call(cnt=None) == E_ARG and call(off=None) == E_ARG
    assert call(rs=None) == E_ARG and call(inv=None) == E_ARG
    assert call(xp=None) == E_ARG
    assert call(H=60) == E_SHAPE
    assert call(x=P_ODD) == E_ALIGN
    assert call(ws=None) == E_WS and call(wsb=ws - 1) == E_WS
    assert call(ws=P_ODD) == E_ALIGN


def test_read_device_error_validation(L):
    import ctypes
    code = ctypes.c_int32(0)
    assert L.moe_read_device_error(None, None, ctypes.byref(code)) == E_ARG
    assert L.moe_read_device_error(P, None, None) == E_ARG
    assert L.moe_read_device_error(P_ODD, None, ctypes.byref(code)) == E_ALIGN


def test_workspaces_hold_the_error_header(L):
    # every workspace size includes the 256-byte error header
    assert L.moe_permute_workspace_bytes(0, 1, 1) >= 256 + 4
    assert L.moe_grouped_ffn_workspace_bytes(64, 4, 128, 128, BF16) >= 256 + 3 * 5 * 4


def test_noalloc_permute_rejects_sizes_beyond_its_scratch(L):
    # 2^30 slots over 256 experts need ~1 GB of scratch: refused on the host
    # before any device call (status 7, MOE_E_SCRATCH)
    st = L.moe_permute_noalloc(P, None, None, 1 << 27, 8, 0, BF16, 256, 0,
                               256, None, None, P, P, P, P, None)
    assert st == 7
    assert L.moe_status_string(7)


def test_ffn_loop_validation(L):
    import ctypes
    f = L.moe_grouped_ffn_loop
    ws = L.moe_grouped_ffn_workspace_bytes(64, 4, 128, 128, BF16)
    hc = (ctypes.c_int32 * 4)(10, 0, 20, 30)
    big = (ctypes.c_int32 * 4)(10, 0, 20, 40)
    neg = (ctypes.c_int32 * 4)(10, -1, 20, 30)

    def call(h=hc, dt=BF16, R=64, x=P):
        return f(x, P, h, None, 4, R, 128, 128, P, P, P, dt, P, P, P, ws, None)

    assert call(h=None) == E_ARG
    assert call(h=big) == E_SHAPE          # 70 rows > R_cap = 64
    assert call(h=neg) == E_SHAPE
    assert call(dt=F32) == 5               # MOE_E_UNSUPPORTED
    assert call(x=P_ODD) == E_ALIGN


def test_ffn_fused_validation(L):
    f = L.moe_grouped_ffn_fused
    ws = L.moe_grouped_ffn_workspace_bytes(64, 4, 128, 128, BF16)

    def call(dt=BF16, R=64, x=P, rs=P, T=32, k=2, H=128, I=128, w=ws, y=P):
        return f(x, rs, T, k, P, None, 4, R, H, I, P, P, P, dt, P, y, P, w, None)

    assert call(dt=F32) == 5               # MOE_E_UNSUPPORTED
    assert call(rs=P, T=16, k=2) == E_SHAPE   # R_cap 64 > T*k = 32
    assert call(rs=P, k=33) == E_SHAPE
    assert call(H=96) == E_SHAPE           # H % 64
    assert call(w=ws - 4) == E_WS
    assert call(y=None) == E_ARG
    assert call(x=P_ODD) == E_ALIGN
    # without row_src, T and k are not used
    assert call(rs=None, T=0, k=0, y=None) == E_ARG


def test_eplb_validation(L):
    f = L.moe_eplb_plan
    assert f(P, 0, 8, 1, P, P, P, P, P, None) == E_SHAPE       # E < 1
    assert f(P, 8, 7, 1, P, P, P, P, P, None) == E_SHAPE       # slots < E
    assert f(P, 8, 10, 4, P, P, P, P, P, None) == E_SHAPE      # 10 % 4 != 0
    assert f(P, 1025, 2048, 2, P, P, P, P, P, None) == E_SHAPE
    assert f(None, 8, 8, 2, P, P, P, P, P, None) == E_ARG
    g = L.moe_permute_replicated
    ws = L.moe_permute_replicated_workspace_bytes(16, 2, 8, 4)
    assert ws > 0
    args = [P, None, None, 16, 2, 0, BF16, 8, 12, P, P, P, P, 0, 4, None, None,
            P, P, P, P, P, ws, None]
    bad = list(args); bad[-2] = ws - 1
    assert g(*bad) == E_WS
    bad = list(args); bad[9] = None
    assert g(*bad) == E_ARG
    bad = list(args); bad[13] = 9                              # s_begin + n_slots > S
    assert g(*bad) == E_SHAPE
    bad = list(args); bad[8] = 7                               # S < E
    assert g(*bad) == E_SHAPE
    h = L.moe_grouped_ffn_slots
    fws = L.moe_grouped_ffn_workspace_bytes(64, 4, 128, 128, BF16)
    assert h(P, P, None, 4, None, 8, 64, 128, 128, P, P, P, BF16, P, P, P, fws, None) == E_ARG
    assert h(P, P, None, 4, P, 8, 64, 128, 128, P, P, P, F32, P, P, P, fws, None) == 5


def test_ffn_validation(L):
    g = L.moe_grouped_gate_up
    # sized for the largest R_cap below (the split-K slots grow with R_cap)
    ws = L.moe_grouped_ffn_workspace_bytes(65, 4, 128, 128, BF16)
    assert ws > L.moe_grouped_ffn_workspace_bytes(64, 4, 128, 128, BF16)

    def call(R=64, H=128, I=128, nl=4, dt=BF16, wsp=P, wsb=ws, x=P, off=P):
        return g(x, off, None, nl, R, H, I, P, P, dt, P, wsp, wsb, None)

    assert call(dt=3) == E_ARG
    assert call(H=96) == E_SHAPE and call(I=100) == E_SHAPE
    assert call(nl=0) == E_SHAPE and call(R=-1) == E_SHAPE
    assert call(off=None) == E_ARG
    assert call(wsp=None) == E_WS and call(wsb=16) == E_WS
    assert call(x=None) == E_ARG
    assert call(x=P_ODD) == E_ALIGN
    assert call(R=0) == 0  # no rows: nothing enqueued
    gg = L.moe_grouped_gate_up_gather

    def gat(x=P, rs=P, T=32, k=2, R=64, dt=BF16):
        return gg(x, rs, T, k, P, None, 4, R, 128, 128, P, P, dt, P, P, ws, None)

    assert gat(dt=F32) == 5                      # MOE_E_UNSUPPORTED
    assert gat(k=0) == E_SHAPE and gat(T=0) == E_SHAPE
    assert gat(R=65) == E_SHAPE                  # R_cap > T * k
    assert gat(rs=None) == E_ARG and gat(x=None) == E_ARG
    assert gat(x=P_ODD) == E_ALIGN
    assert gat(R=0) == 0
    d = L.moe_grouped_down
    assert d(P, P, 4, 64, 100, 128, P, BF16, P, P, ws, None) == E_SHAPE
    assert d(P, P, 4, 64, 128, 128, None, BF16, P, P, ws, None) == E_ARG
    # the grouped FFN as one call (bf16: one plan kernel), and its gather
    # variant
    ff = L.moe_grouped_ffn

    def ffn(x=P, wd=P, y=P, dt=BF16, R=64, wsb=ws):
        return ff(x, P, None, 4, R, 128, 128, P, P, wd, dt, P, y, P, wsb, None)

    assert ffn(wd=None) == E_ARG and ffn(y=None) == E_ARG
    assert ffn(x=None) == E_ARG
    assert ffn(x=P_ODD) == E_ALIGN and ffn(y=P_ODD) == E_ALIGN
    assert ffn(wsb=16) == E_WS
    assert ffn(R=0) == 0
    fg = L.moe_grouped_ffn_gather

    def fga(x=P, rs=P, T=32, k=2, R=64, dt=BF16, wd=P, y=P, wsb=ws):
        return fg(x, rs, T, k, P, None, 4, R, 128, 128, P, P, wd, dt, P, y, P,
                  wsb, None)

    assert fga(dt=F32) == 5                      # MOE_E_UNSUPPORTED
    assert fga(k=0) == E_SHAPE and fga(T=0) == E_SHAPE and fga(k=33) == E_SHAPE
    assert fga(R=65) == E_SHAPE                  # R_cap > T * k
    assert fga(rs=None) == E_ARG and fga(wd=None) == E_ARG
    assert fga(y=None) == E_ARG and fga(x=None) == E_ARG
    assert fga(x=P_ODD) == E_ALIGN and fga(y=P_ODD) == E_ALIGN
    assert fga(wsb=16) == E_WS
    assert fga(R=0) == 0


def test_combine_validation(L):
    c = L.moe_unpermute_combine
    assert c(P, P, None, 8, 2, 12, BF16, P, None) == E_SHAPE
    assert c(P, P, None, 8, 0, 16, BF16, P, None) == E_SHAPE
    assert c(P, P, None, 8, 2, 16, 9, P, None) == E_ARG
    assert c(P_ODD, P, None, 8, 2, 16, BF16, P, None) == E_ALIGN
    assert c(None, P, None, 8, 2, 16, BF16, P, None) == E_ARG
    assert c(None, None, None, 0, 2, 16, BF16, None, None) == 0


def test_mxfp8_validation(L):
    q = L.moe_mxfp8_quantize
    # axis, format, cols % 32, alignment, align value, capacity, segments
    # need pad
    assert q(P, 64, 64, 64, 2, 0, None, 0, 32, P, 64, P, 2, None, None) == E_ARG
    assert q(P, 64, 64, 64, 0, 2, None, 0, 32, P, 64, P, 2, None, None) == E_ARG
    assert q(P, 64, 48, 48, 0, 0, None, 0, 32, P, 48, P, 2, None, None) == E_SHAPE
    assert q(P, 64, 64, 64, 0, 1, None, 0, 32, P_ODD, 64, P, 2, None, None) == E_ALIGN
    assert q(P, 64, 64, 64, 1, 0, None, 0, 16, P, 64, P, 2, None, None) == E_SHAPE
    assert q(P, 64, 64, 64, 1, 0, None, 0, 32, P, 48, P, 2, None, None) == E_SHAPE
    assert q(P, 64, 64, 64, 1, 0, P, 2, 32, P, 128, P, 4, None, None) == E_ARG
    assert q(P, 64, 64, 64, 1, 1, P, 2, 32, P, 80, P, 4, P, None) == E_SHAPE
    assert q(P, 0, 64, 64, 0, 1, None, 0, 32, P, 64, P, 2, None, None) == 0

    fb = L.moe_grouped_mlp_mxfp8_fwd_workspace_bytes
    assert fb(100, 4, 512, 512) > 0 and fb(100, 4, 500, 512) == 0
    assert fb(100, 4, 512, 256) == 0 and fb(100, 0, 512, 512) == 0
    ws = fb(64, 2, 512, 512)
    f = L.moe_grouped_mlp_mxfp8_fwd

    def fwd(H=512, I=512, xq=P, wsp=P, wsb=ws, R=64):
        return f(xq, P, P, None, 2, R, H, I, P, P, P, P, P, P, P, P, P, wsp,
                 wsb, None)

    assert fwd(H=256) == E_SHAPE and fwd(I=520) == E_SHAPE
    assert fwd(xq=None) == E_ARG and fwd(xq=P_ODD) == E_ALIGN
    assert fwd(wsp=None) == E_WS and fwd(wsb=ws - 1) == E_WS
    assert fwd(R=0) == 0

    fd = L.moe_grouped_mlp_mxfp8_fwd_down
    assert fd(P, 2, 64, 256, 512, P, P, P, P, ws, None) == E_SHAPE
    assert fd(None, 2, 64, 512, 512, P, P, P, P, ws, None) == E_ARG
    assert fd(P, 2, 64, 512, 512, P, P, P_ODD, P, ws, None) == E_ALIGN
    assert fd(P, 2, 64, 512, 512, P, P, P, P, ws - 1, None) == E_WS
    assert fd(P, 2, 0, 512, 512, P, P, P, P, ws, None) == 0

    lb = L.moe_grouped_linear_mxfp8_workspace_bytes(64, 2, 1024)
    assert lb > 0 and L.moe_grouped_linear_mxfp8_workspace_bytes(64, 2, 1000) == 0
    g = L.moe_grouped_linear_mxfp8
    assert g(P, P, 2, 64, 1024, 0, P, P, P, P, lb, None) == E_SHAPE
    assert g(P, P, 2, 64, 1000, 64, P, P, P, P, lb, None) == E_SHAPE
    assert g(P, None, 2, 64, 1024, 64, P, P, P, P, lb, None) == E_ARG
    assert g(P, P, 2, 64, 1024, 64, P, P, P_ODD, P, lb, None) == E_ALIGN
    assert g(P, P, 2, 64, 1024, 64, P, P, P, P, lb - 1, None) == E_WS

    db = L.moe_grouped_mlp_mxfp8_bwd_down_workspace_bytes(64, 2, 512, 512)
    gb = L.moe_grouped_mlp_mxfp8_bwd_gate_up_workspace_bytes(64, 2, 512, 512)
    bb = L.moe_grouped_mlp_mxfp8_bwd_workspace_bytes(64, 2, 512, 512)
    # the fused call keeps the MX codes of [dg | du] beside the down workspace
    assert db > 0 and gb > 0 and bb >= db + 64 * 2 * 512
    d = L.moe_grouped_mlp_mxfp8_bwd_down
    assert d(P, None, P, None, 2, 64, 512, 512, P, P, P, P, P, 0, P, db, None) == E_ARG
    assert d(P, P, P, None, 2, 64, 512, 512, P, P, P, P, P, 0, P, db - 1, None) == E_WS
    assert d(P, P, P, None, 2, 64, 512, 512, P, P, P, P, P, 2, P, db, None) == E_ARG
    u = L.moe_grouped_mlp_mxfp8_bwd_gate_up
    assert u(P, P, P, 2, 64, 512, 512, P, P, P, P, None, P, P, 0, P, gb, None) == E_ARG
    assert u(P, P, P, 2, 64, 512, 512, P, P, P, P, P, P, P_ODD, 1, P, gb, None) == E_ALIGN
    assert u(P, P, P, 2, 64, 512, 512, P, P, P, P, P, P, P, 1, P, gb - 1, None) == E_WS
    assert u(P, P, P, 2, 64, 512, 512, P, P, P, P, P, P, P, -1, P, gb, None) == E_ARG
    b = L.moe_grouped_mlp_mxfp8_bwd
    args = [P, P, P, P, None, 2, 64, 512, 512] + [P] * 11 + [0, P, bb, None]
    bad = list(args); bad[-2] = bb - 1
    assert b(*bad) == E_WS
    bad = list(args); bad[0] = None
    assert b(*bad) == E_ARG
    bad = list(args); bad[-4] = 5
    assert b(*bad) == E_ARG


def _py_sources(d):
    for root, _, files in os.walk(os.path.join(ROOT, d)):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h", ".c")):
                yield os.path.join(root, fn)


def test_product_and_oracle_share_nothing():
    pat_oracle = re.compile(r"^\s*(import|from)\s+oracle\b|moe_oracle|libmoe_oracle", re.M)
    for path in _py_sources("mixture_experts_expert_router_amd"):
        assert not pat_oracle.search(open(path, encoding="utf-8").read()), path
    pat_pkg = re.compile(r"mixture_experts_expert_router_amd|moe_mi355x|csrc/")
    for path in _py_sources("oracle"):
        assert not pat_pkg.search(open(path, encoding="utf-8").read()), path
