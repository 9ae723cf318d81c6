"""MXFP8 path through the C ABI against the CPU oracle.

Codes and scales of given bf16 inputs must match bit for bit.  Float
outputs must meet max(|err| - storage slack) <= 6e-2 * RMS of each row of
the reference (the oracle dequantises exactly and works in fp64; the slack
is one bf16 ulp of the element for bf16 outputs, none for fp32 ones).

The fused forward and backward are checked end to end against the plain
oracle step, in which every tensor of the chain (a, g, u, dg, du) is
quantised from its unrounded value (fp32 on the device, fp64 in the
oracle).  Such a quantisation is floating point deciding an integer on
values the two sides compute differently, so (mx_check):
  - the computed values are compared element by element: g, u, a, ds (and,
    through the stage call, dg, du);
  - every MX code and scale the device chose (read from the workspace
    through moe_mxfp8_workspace_view) must be the rule's rounding of a
    value within TAU_DEC * RMS(row) of the oracle's;
  - every output of a GEMM that consumes those codes (y, dX, dW_gate,
    dW_up, dW_down) is compared element by element with the oracle's exact
    product of the device's codes and the oracle's own quantisation of the
    other operand.
The unfused stage calls are checked against the oracle's stage functions on
the same given inputs; the backward stages hand [dg | du] on in bf16, which
the oracle's labelled bf16_dgu variant models.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_router_amd as moe
import moe_synth as synth
import oracle as orc
from gpu_util import print_case, rel_err, scaled_excess, to_dev, to_f64
from mx_check import check_block_decisions, dequantize, segment_columns

pytestmark = pytest.mark.gpu
TAU = 6e-2
TAU_DEC = 1e-3     # admissible distance of a decided value, * RMS(row)


def bf16_bits(a):
    t = torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def special_rows(cols, rng):
    rows = [rng.standard_normal(cols) * 10.0 ** rng.integers(-3, 3)]
    z = np.zeros(cols); rows.append(z)                            # all-zero block
    p2 = 2.0 ** rng.integers(-20, 20, cols) * rng.choice([-1, 1], cols)
    rows.append(p2)                                               # powers of two
    mid = np.full(cols, 448.0); mid[1::2] = 1.0625 * 2 ** 0       # ties after scaling
    rows.append(mid)
    tiny = rng.standard_normal(cols); tiny[::3] = -1e-30          # rounds to -0
    rows.append(tiny)
    big = rng.standard_normal(cols) * 1e30; rows.append(big)
    return np.stack(rows)


def test_quantize_rows_bit_exact():
    rng = np.random.default_rng(5)
    cols = 256
    v = np.concatenate([rng.standard_normal((61, cols)), special_rows(cols, rng)])
    xb = bf16_bits(v)
    codes, scales = moe.mxfp8_quantize(to_dev(xb), 0)
    moe.debug_sync()
    rc, rs = orc.mx_quantize_rows(orc.to_f64(xb))
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("align", [32, 512])
def test_quantize_cols_segments_bit_exact(align):
    rng = np.random.default_rng(6)
    rows, cols = 100, 96
    xb = bf16_bits(rng.standard_normal((rows, cols)))
    seg = np.array([0, 5, 5, 70, 100], dtype=np.int32)
    codes, scales, pad = moe.mxfp8_quantize(to_dev(xb), 1, to_dev(seg), align)
    moe.debug_sync()
    pad = pad.cpu().numpy()
    lens = np.diff(seg)
    np.testing.assert_array_equal(pad, np.concatenate([[0], np.cumsum((lens + align - 1) // align * align)]))
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    x64 = orc.to_f64(xb)
    for i in range(len(seg) - 1):
        n = seg[i + 1] - seg[i]
        if n == 0:
            continue
        npad = (n + align - 1) // align * align
        blk = np.zeros((cols, npad))
        blk[:, :n] = x64[seg[i]:seg[i + 1]].T
        rc, rs = orc.mx_quantize_rows(blk)
        np.testing.assert_array_equal(c[:, pad[i]:pad[i] + npad], rc)
        np.testing.assert_array_equal(s[:, pad[i] // 32:(pad[i] + npad) // 32], rs)


def exhaustive_blocks():
    """Blocks of 32 bf16 bit patterns that put every finite bf16 value under
    every shared exponent X = -127..119.  For each biased bf16 exponent eb
    (0..254) the anchor is the largest magnitude with that exponent
    (mantissa 0x7F), which fixes the block's X (clamped to -127 for small
    eb); the other 31 slots run through every magnitude up to the anchor, with
    both signs.  Two all-zero blocks (+0, -0) close the list.  Returns
    [n, 32] uint16, n a multiple of 1024."""
    out = []
    for eb in range(255):
        a = (eb << 7) | 0x7F
        mags = np.arange(a + 1, dtype=np.uint16)
        vals = np.concatenate([mags, mags | np.uint16(0x8000)])
        n = -(-len(vals) // 31)
        vals = np.concatenate([vals, np.zeros(n * 31 - len(vals), np.uint16)])
        b = np.empty((n, 32), np.uint16)
        b[:, 0] = a | (0x8000 if eb & 1 else 0)
        b[:, 1:] = vals.reshape(n, 31)
        out.append(b)
    out.append(np.zeros((1, 32), np.uint16))
    out.append(np.full((1, 32), 0x8000, np.uint16))
    blk = np.concatenate(out)
    pad = -len(blk) % 1024
    return np.concatenate([blk, np.zeros((pad, 32), np.uint16)])


@pytest.fixture(scope="module")
def exhaustive():
    blk = exhaustive_blocks()
    print_case("exhaustive quantisation blocks", blk.shape[0])
    rc, rs = orc.mx_quantize_rows(orc.to_f64(blk))
    return blk, rc, rs.reshape(-1)


@pytest.mark.timeout(300)
def test_quantize_rows_every_bf16_at_every_scale(exhaustive):
    blk, rc, rs = exhaustive
    C = 1024                                       # 32 blocks per row
    x = np.ascontiguousarray(blk.reshape(-1, C))
    codes, scales = moe.mxfp8_quantize(to_dev(x), 0)
    moe.debug_sync()
    np.testing.assert_array_equal(scales.cpu().numpy().reshape(-1), rs)
    np.testing.assert_array_equal(codes.cpu().numpy().reshape(-1, 32), rc)


@pytest.mark.timeout(300)
def test_quantize_cols_every_bf16_at_every_scale(exhaustive):
    blk, rc, rs = exhaustive
    C = 1024                                       # block g*C + c -> column c
    g = blk.shape[0] // C
    x = np.ascontiguousarray(blk.reshape(g, C, 32).transpose(0, 2, 1).reshape(g * 32, C))
    codes, scales, _ = moe.mxfp8_quantize(to_dev(x), 1)
    moe.debug_sync()
    np.testing.assert_array_equal(
        codes.cpu().numpy(), rc.reshape(g, C, 32).transpose(1, 0, 2).reshape(C, g * 32))
    np.testing.assert_array_equal(scales.cpu().numpy(), rs.reshape(g, C).T)


def _mx_case(name):
    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl)
    idx, w = orc.topk_softmax(inp["logits"], wl.k)
    p = orc.permute(idx, 0, wl.n_local)
    x_perm = orc.gather_rows(inp["x"], p["row_src"], wl.k)
    s = w.reshape(-1)[p["row_src"]].astype(np.float32)
    dy = synth.make_dy(wl, p["R"])
    ref = orc.mxfp8_mlp_step(x_perm, p["offsets"], s.astype(np.float64),
                             inp["w_gate"], inp["w_up"], inp["w_down"], dy)
    return wl, inp, p, x_perm, s, dy, ref


def _bits(v):
    """bf16 bits of the nearest bf16 values of v."""
    v = orc.round_bf16(v)
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _check(got, ref, what, bad, dtype="bf16"):
    e = scaled_excess(got, ref, dtype)
    print_case(what, f"row excess {e:.2e}, plain {rel_err(got, ref):.2e}")
    if not e <= TAU:
        bad.append(f"{what}: {e:.3e}")


def _ds(t, R):
    return t[:R].cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module", params=["small_mxfp8", "mid_mxfp8"])
def case(request):
    name = request.param
    print_case(name)
    wl, inp, p, x_perm, s, dy, ref = _mx_case(name)
    d = {k: to_dev(inp[k]) for k in ("w_gate", "w_up", "w_down")}
    mw = moe.MxWeights(d["w_gate"], d["w_up"], d["w_down"])
    return dict(name=name, wl=wl, inp=inp, p=p, x_perm=x_perm, s=s, dy=dy,
                ref=ref, mw=mw, offs=to_dev(p["offsets"]), st=to_dev(s))


def _ws(n, dev="cuda"):
    return torch.empty(max(n, 16), dtype=torch.uint8, device=dev)


def _run_fused(c, x_perm=None, offs=None, st=None, mw=None, dy=None, gf="e4m3"):
    """Fused forward (one call) and fused backward (gradient operands in
    format gf), keeping the workspaces."""
    xt = to_dev(c["x_perm"] if x_perm is None else x_perm)
    xq, xs = moe.mxfp8_quantize(xt, 0)
    offs = c["offs"] if offs is None else offs
    st = c["st"] if st is None else st
    mw = c["mw"] if mw is None else mw
    R_cap, H = xt.shape
    L = moe.lib()
    ws_f = _ws(L.moe_grouped_mlp_mxfp8_fwd_workspace_bytes(R_cap, mw.n_local, H, mw.I))
    ws_b = _ws(L.moe_grouped_mlp_mxfp8_bwd_workspace_bytes(R_cap, mw.n_local, H, mw.I))
    a, gu, y = moe.mxfp8_mlp_fwd(xq, xs, offs, st, mw, workspace=ws_f)
    g = moe.mxfp8_mlp_bwd(to_dev(c["dy"] if dy is None else dy), xt, gu, offs,
                          st, mw, workspace=ws_b, grad_format=gf)
    return dict(xt=xt, a=a, gu=gu, y=y, g=g, ws_f=ws_f, ws_b=ws_b, R_cap=R_cap)


def _rows_delta(v):
    rms = np.sqrt(np.mean(np.asarray(v, np.float64) ** 2, axis=1, keepdims=True))
    return np.broadcast_to(TAU_DEC * rms, np.shape(v))


def _decisions(what, v, delta, codes, scales, bad, fmt="e4m3"):
    bs, bc, differ = check_block_decisions(v, delta, codes, scales, fmt)
    print_case(what, f"codes differing from the oracle's {differ} of {np.size(v)}, "
               f"inadmissible scales {bs}, codes {bc}")
    if bs or bc:
        bad.append(f"{what}: {bs} scales, {bc} codes inadmissible")


def _verify_fused(c, run, ref, offsets, wl, tag, bad, experts=None, gf="e4m3"):
    """The checks of the module docstring on one fused forward + backward
    (gradient codes in format gf)."""
    R, H, I, n = int(offsets[-1]), wl.H, wl.I, wl.n_local
    inp = c["inp"]
    a, gu, y, g = run["a"], run["gu"], run["y"], run["g"]
    experts = range(n) if experts is None else experts
    live = [e for e in range(n) if offsets[e + 1] > offsets[e]]
    # computed values
    _check(to_f64(gu[:R, :I]), ref["g"], f"{tag} g", bad, "f32")
    _check(to_f64(gu[:R, I:]), ref["u"], f"{tag} u", bad, "f32")
    _check(to_f64(a[:R]), ref["a"], f"{tag} a", bad)
    _check(_ds(g["ds"], R), ref["ds"], f"{tag} ds", bad, "f32")
    # forward: MX(a) decisions, then y from the device's codes
    aq, as_, _ = moe.mxfp8_workspace_view(run["ws_f"], moe.MXCALL_FWD, moe.MXT_A_ROWS,
                                          run["R_cap"], n, H, I)
    aq, as_ = aq[:R].cpu().numpy(), as_[:R].cpu().numpy()
    _decisions(f"{tag} MX(a)", ref["a"], _rows_delta(ref["a"]), aq, as_, bad)
    a_dev = dequantize(aq, as_)
    y_ref = np.zeros((R, H))
    for e in live:
        sl = slice(int(offsets[e]), int(offsets[e + 1]))
        y_ref[sl] = orc.matmul_nt(a_dev[sl], orc.mx_roundtrip_rows(orc.to_f64(inp["w_down"][e])))
    _check(to_f64(y[:R]), y_ref, f"{tag} y (device codes)", bad)
    print_case(f"{tag} y against the plain oracle",
               f"row excess {scaled_excess(to_f64(y[:R]), ref['y'], 'bf16'):.2e}")
    # backward: [dg | du] row-wise decisions, then dX from the device's codes
    view = lambda t: moe.mxfp8_workspace_view(run["ws_b"], moe.MXCALL_BWD, t,
                                              run["R_cap"], n, H, I)
    dgu = np.concatenate([ref["dg"], ref["du"]], axis=1)
    q, qs, _ = view(moe.MXT_DGU_ROWS)
    q, qs = q[:R].cpu().numpy(), qs[:R].cpu().numpy()
    _decisions(f"{tag} MX([dg | du]) rows", dgu, _rows_delta(dgu), q, qs, bad, gf)
    d_dev = dequantize(q, qs, gf)
    dx_ref = np.zeros((R, H))
    for e in live:
        sl = slice(int(offsets[e]), int(offsets[e + 1]))
        wg = orc.mx_roundtrip_rows(np.ascontiguousarray(orc.to_f64(inp["w_gate"][e]).T))
        wu = orc.mx_roundtrip_rows(np.ascontiguousarray(orc.to_f64(inp["w_up"][e]).T))
        dx_ref[sl] = orc.matmul_nt(d_dev[sl, :I], wg) + orc.matmul_nt(d_dev[sl, I:], wu)
    _check(to_f64(g["dx"][:R]), dx_ref, f"{tag} dx (device codes)", bad)
    # column-wise decisions of dg, du, then dW_gate, dW_up from them
    xf = orc.to_f64(c["x_perm"][:R])
    for key, t, vref in (("dw_gate", moe.MXT_DG_COLS, ref["dg"]),
                         ("dw_up", moe.MXT_DU_COLS, ref["du"])):
        cq, cs, pad = view(t)
        cq, cs, pad = cq.cpu().numpy(), cs.cpu().numpy(), pad.cpu().numpy()
        W = int(pad[-1])
        vt = segment_columns(vref, offsets, pad, W)
        dt = segment_columns(_rows_delta(vref), offsets, pad, W)
        _decisions(f"{tag} MX({key[3:]}) columns", vt, dt, cq[:, :W], cs, bad, gf)
        c_dev = dequantize(cq[:, :W], cs, gf)
        for e in experts:
            r0, r1 = int(offsets[e]), int(offsets[e + 1])
            if r1 == r0:
                continue
            qx = orc.mx_roundtrip_rows(np.ascontiguousarray(xf[r0:r1].T))   # [H, n_e]
            wref = orc.matmul_nt(c_dev[:, pad[e]:pad[e] + (r1 - r0)], qx)
            _check(to_f64(g[key][e]), wref, f"{tag} {key}[{e}] (device codes)", bad)


def test_mxfp8_fused_forward_backward(case):
    """Every output of the fused forward and backward against the plain
    oracle step, by the rule of the module docstring; dW_down through the
    stage call, whose bits the fused call's equal."""
    c, ref, R, I = case, case["ref"], case["p"]["R"], case["wl"].I
    run = _run_fused(c)
    moe.debug_sync()
    bad = []
    _verify_fused(c, run, ref, c["p"]["offsets"], c["wl"], c["name"], bad)
    _verify_dw_down(c, run, ref, c["p"]["offsets"], c["wl"], c["name"], bad)
    assert not bad, bad


def _verify_dw_down(c, run, ref, offsets, wl, tag, bad, experts=None, gf="e4m3"):
    """dW_down: the stage call (same epilogue and codes as the fused call,
    which it must equal bit for bit) leaves the column-wise MX(a) in its
    workspace; check those decisions against the oracle's a, then dW_down
    against the exact product of the oracle's MX(dY) and the device's MX(a)."""
    R, H, I, n = int(offsets[-1]), wl.H, wl.I, wl.n_local
    R_cap = run["R_cap"]
    ws = _ws(moe.lib().moe_grouped_mlp_mxfp8_bwd_down_workspace_bytes(R_cap, n, H, I))
    d1 = moe.mxfp8_mlp_bwd_down(to_dev(c["dy"]), run["gu"], c["offs"], c["st"],
                                c["mw"], workspace=ws, grad_format=gf)
    moe.debug_sync()
    assert torch.equal(d1["dw_down"], run["g"]["dw_down"]), f"{tag} stage dw_down"
    assert torch.equal(d1["ds"][:R], run["g"]["ds"][:R]), f"{tag} stage ds"
    cq, cs, pad = moe.mxfp8_workspace_view(ws, moe.MXCALL_BWD_DOWN, moe.MXT_A_COLS,
                                           R_cap, n, H, I)
    cq, cs, pad = cq.cpu().numpy(), cs.cpu().numpy(), pad.cpu().numpy()
    W = int(pad[-1])
    _decisions(f"{tag} MX(a) columns", segment_columns(ref["a"], offsets, pad, W),
               segment_columns(_rows_delta(ref["a"]), offsets, pad, W), cq[:, :W], cs, bad)
    a_dev = dequantize(cq[:, :W], cs)
    dyf = orc.to_f64(c["dy"][:R])
    for e in (range(n) if experts is None else experts):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        qdy = orc.mx_roundtrip_rows(np.ascontiguousarray(dyf[r0:r1].T), gf)  # [H, n_e]
        wref = orc.matmul_nt(qdy, a_dev[:, pad[e]:pad[e] + (r1 - r0)])
        _check(to_f64(d1["dw_down"][e]), wref, f"{tag} dw_down[{e}] (device codes)", bad)


def test_mxfp8_down_projection_stage(case):
    """moe_grouped_linear_mxfp8 on a given bf16 a: y = Q_I(a) Q_I(W_d)^T."""
    c, ref, R = case, case["ref"], case["p"]["R"]
    ab = _bits(ref["a"])
    y = moe.grouped_linear_mxfp8(to_dev(ab), c["offs"], c["wl"].n_local,
                                 c["mw"].wd, c["mw"].wds)
    moe.debug_sync()
    off = c["p"]["offsets"]
    y_ref = np.zeros((R, c["wl"].H))
    for e in range(c["wl"].n_local):
        sl = slice(int(off[e]), int(off[e + 1]))
        if sl.stop > sl.start:
            y_ref[sl] = orc.mx_gemm_nt(orc.to_f64(ab[sl]),
                                       orc.to_f64(c["inp"]["w_down"][e]))
    bad = []
    _check(to_f64(y[:R]), y_ref, f"{c['name']} stage y", bad)
    assert not bad, bad


def test_mxfp8_backward_down_stage(case):
    """moe_grouped_mlp_mxfp8_bwd_down on given fp32 g, u (the oracle's,
    rounded to fp32) against the oracle's down/SwiGLU backward on the same
    values: dg, du (bf16 outputs), ds, dW_down."""
    c, ref, R, I = case, case["ref"], case["p"]["R"], case["wl"].I
    g32 = ref["g"].astype(np.float32)
    u32 = ref["u"].astype(np.float32)
    gu = np.ascontiguousarray(np.concatenate([g32, u32], axis=1))
    out = moe.mxfp8_mlp_bwd_down(to_dev(c["dy"]), to_dev(gu), c["offs"],
                                 c["st"], c["mw"])
    moe.debug_sync()
    sref = orc.mxfp8_backward_down(c["dy"], g32, u32, c["s"].astype(np.float64),
                                   c["p"]["offsets"], c["inp"]["w_down"])
    bad = []
    n = c["name"]
    _check(to_f64(out["dgu"][:R, :I]), sref["dg"], f"{n} stage dg", bad)
    _check(to_f64(out["dgu"][:R, I:]), sref["du"], f"{n} stage du", bad)
    _check(_ds(out["ds"], R), sref["ds"], f"{n} stage ds", bad, "f32")
    for e in range(c["wl"].n_local):
        _check(to_f64(out["dw_down"][e]), sref["dw_down"][e],
               f"{n} stage dw_down[{e}]", bad)
    assert not bad, bad


def test_mxfp8_backward_gate_up_stage(case):
    """moe_grouped_mlp_mxfp8_bwd_gate_up on a given bf16 [dg | du] (the
    oracle's dg, du rounded) against the oracle step's bf16_dgu variant,
    which quantises the same bf16 values."""
    c, ref, R, I = case, case["ref"], case["p"]["R"], case["wl"].I
    dg_b, du_b = _bits(ref["dg"]), _bits(ref["du"])
    dgu = np.concatenate([dg_b, du_b], axis=1)
    out = moe.mxfp8_mlp_bwd_gate_up(to_dev(dgu), to_dev(c["x_perm"]),
                                    c["offs"], c["mw"])
    moe.debug_sync()
    # the oracle step's labelled variant for this API: [dg | du] rounded
    # to bf16 before the gate/up backward quantises it
    sref = orc.mxfp8_mlp_step(c["x_perm"], c["p"]["offsets"],
                              c["s"].astype(np.float64), c["inp"]["w_gate"],
                              c["inp"]["w_up"], c["inp"]["w_down"], c["dy"],
                              bf16_dgu=True)
    bad = []
    n = c["name"]
    _check(to_f64(out["dx"][:R]), sref["dx"], f"{n} stage dx", bad)
    for key in ("dw_gate", "dw_up"):
        for e in range(c["wl"].n_local):
            _check(to_f64(out[key][e]), sref[key][e], f"{n} stage {key}[{e}]", bad)
    assert not bad, bad


def test_mxfp8_fused_and_stage_calls_agree(case):
    """Structural identities: the two-call forward (gate/up, then the down
    projection from the workspace codes) equals the one-call forward bit for
    bit, and the fused backward's ds and dW_down equal the stage call's
    (the same epilogue and the same codes)."""
    c, R = case, case["p"]["R"]
    wl = c["wl"]
    run = _run_fused(c)
    xt, R_cap = run["xt"], run["R_cap"]
    xq, xs = moe.mxfp8_quantize(xt, 0)
    ws = _ws(moe.lib().moe_grouped_mlp_mxfp8_fwd_workspace_bytes(R_cap, wl.n_local, wl.H, wl.I))
    moe.mxfp8_mlp_fwd(xq, xs, c["offs"], c["st"], c["mw"], workspace=ws, down=False)
    y_two = moe.mxfp8_mlp_fwd_down(c["offs"], c["mw"], ws, R_cap)
    d1 = moe.mxfp8_mlp_bwd_down(to_dev(c["dy"]), run["gu"], c["offs"], c["st"], c["mw"])
    moe.debug_sync()
    print_case(c["name"], "fused vs stage calls, rows", R)
    assert torch.equal(run["y"][:R], y_two[:R])
    assert torch.equal(run["g"]["ds"][:R], d1["ds"][:R])
    assert torch.equal(run["g"]["dw_down"], d1["dw_down"])


def _seg_case(counts, seed):
    wl = synth.WORKLOADS["small_mxfp8"]
    R = sum(counts)
    inp = synth.make_inputs(wl, tokens=R)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x_perm = inp["x"]
    s = np.random.default_rng(seed).uniform(0.05, 1.0, R).astype(np.float32)
    dy = synth.make_dy(wl, R)
    ref = orc.mxfp8_mlp_step(x_perm, offsets, s.astype(np.float64),
                             inp["w_gate"], inp["w_up"], inp["w_down"], dy)
    d = {k: to_dev(inp[k]) for k in ("w_gate", "w_up", "w_down")}
    mw = moe.MxWeights(d["w_gate"], d["w_up"], d["w_down"])
    c = dict(x_perm=x_perm, dy=dy, offs=to_dev(offsets), st=to_dev(s), mw=mw,
             inp=inp)
    return wl, R, ref, c


@pytest.mark.parametrize("counts", [
    [0, 127, 0, 173],        # experts 0 and 2 receive no rows
    [3, 0, 1, 37],           # tiny ragged segments: tiles mostly padding
])
def test_mxfp8_ragged_and_empty_segments(counts):
    """Experts without rows get exact zero weight gradients; with 1-37 rows
    per expert a weight-gradient block holds few values, and every output
    still meets the oracle row by row."""
    wl, R, ref, c = _seg_case(counts, 11)
    print_case("small_mxfp8 segments", counts)
    run = _run_fused(c)
    moe.debug_sync()
    g = run["g"]
    for key in ("dw_gate", "dw_up", "dw_down"):
        for e, n in enumerate(counts):
            if n == 0:
                assert not g[key][e].any(), (key, e)
    bad = []
    live = [e for e, n in enumerate(counts) if n > 0]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    tag = f"segments {counts}"
    _verify_fused(c, run, ref, offsets, wl, tag, bad, experts=live)
    _verify_dw_down(c, run, ref, offsets, wl, tag, bad, experts=live)
    assert not bad, bad


def test_mxfp8_step_captured_in_a_graph_replays_bit_exactly(case):
    """Quantise x, fused forward, fused backward captured in one HIP graph:
    every replay (eager work and synchronisation between them) equals the
    eager step bit for bit."""
    c, R = case, case["p"]["R"]
    wl = c["wl"]
    xt = to_dev(c["x_perm"])
    dyt = to_dev(c["dy"])
    R_cap, H = xt.shape
    I, n = wl.I, wl.n_local
    bf = torch.bfloat16
    dev = xt.device
    xq = torch.empty((R_cap, H), dtype=torch.uint8, device=dev)
    xs = torch.empty((R_cap, H // 32), dtype=torch.uint8, device=dev)
    a = torch.empty((R_cap, I), dtype=bf, device=dev)
    gu = torch.empty((R_cap, 2 * I), dtype=torch.float32, device=dev)
    y = torch.empty((R_cap, H), dtype=bf, device=dev)
    outs = dict(dx=torch.empty((R_cap, H), dtype=bf, device=dev),
                ds=torch.empty(R_cap, dtype=torch.float32, device=dev),
                dw_gate=torch.empty((n, I, H), dtype=bf, device=dev),
                dw_up=torch.empty((n, I, H), dtype=bf, device=dev),
                dw_down=torch.empty((n, H, I), dtype=bf, device=dev))
    L = moe.lib()
    ws_f = torch.empty(L.moe_grouped_mlp_mxfp8_fwd_workspace_bytes(R_cap, n, H, I),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(L.moe_grouped_mlp_mxfp8_bwd_workspace_bytes(R_cap, n, H, I),
                       dtype=torch.uint8, device=dev)

    def step():
        moe.mxfp8_quantize(xt, 0, codes=xq, scales=xs)
        moe.mxfp8_mlp_fwd(xq, xs, c["offs"], c["st"], c["mw"], a=a, gu=gu, y=y,
                          workspace=ws_f)
        moe.mxfp8_mlp_bwd(dyt, xt, gu, c["offs"], c["st"], c["mw"],
                          workspace=ws_b, **outs)

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    ref["y"] = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    print_case(c["name"], "graph replays")
    for rep in range(3):
        for v in outs.values():
            v.zero_()
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y[:R], ref["y"][:R]), rep
        assert torch.equal(outs["dx"][:R], ref["dx"][:R]), rep
        assert torch.equal(outs["ds"][:R], ref["ds"][:R]), rep
        for key in ("dw_gate", "dw_up", "dw_down"):
            assert torch.equal(outs[key], ref[key]), (rep, key)
        _ = (xt.float().sum() + dyt.float().sum()).item()


# ---------------------------------------------------------------- E5M2 gradients


@pytest.fixture(scope="module")
def exhaustive5():
    blk = exhaustive_blocks()
    rc, rs = orc.mx_quantize_rows(orc.to_f64(blk), "e5m2")
    return blk, rc, rs.reshape(-1)


@pytest.mark.timeout(300)
def test_quantize_e5m2_every_bf16_at_every_scale(exhaustive5):
    """Every finite bf16 value under every E5M2 shared exponent, through the
    row and the column quantiser, bit for bit against the oracle."""
    blk, rc, rs = exhaustive5
    C = 1024
    print_case("exhaustive E5M2 quantisation blocks", blk.shape[0])
    x = np.ascontiguousarray(blk.reshape(-1, C))
    codes, scales = moe.mxfp8_quantize(to_dev(x), 0, fmt="e5m2")
    g = blk.shape[0] // C
    xc = np.ascontiguousarray(blk.reshape(g, C, 32).transpose(0, 2, 1).reshape(g * 32, C))
    ccodes, cscales, _ = moe.mxfp8_quantize(to_dev(xc), 1, fmt="e5m2")
    moe.debug_sync()
    np.testing.assert_array_equal(scales.cpu().numpy().reshape(-1), rs)
    np.testing.assert_array_equal(codes.cpu().numpy().reshape(-1, 32), rc)
    np.testing.assert_array_equal(
        ccodes.cpu().numpy(), rc.reshape(g, C, 32).transpose(1, 0, 2).reshape(C, g * 32))
    np.testing.assert_array_equal(cscales.cpu().numpy(), rs.reshape(g, C).T)


def _ref5(c):
    if "ref5" not in c:
        c["ref5"] = orc.mxfp8_mlp_step(c["x_perm"], c["p"]["offsets"],
                                       c["s"].astype(np.float64), c["inp"]["w_gate"],
                                       c["inp"]["w_up"], c["inp"]["w_down"], c["dy"],
                                       grad_fmt="e5m2")
    return c["ref5"]


def test_mxfp8_fused_backward_e5m2_gradients(case):
    """The fused backward with dY, dg, du in E5M2 against the oracle step
    with grad_fmt="e5m2", by the rule of the module docstring (decisions of
    the [dg | du] codes in E5M2, every GEMM output from the device's codes)."""
    c = case
    ref = _ref5(c)
    run = _run_fused(c, gf="e5m2")
    moe.debug_sync()
    bad = []
    tag = f"{c['name']} e5m2"
    _verify_fused(c, run, ref, c["p"]["offsets"], c["wl"], tag, bad, gf="e5m2")
    _verify_dw_down(c, run, ref, c["p"]["offsets"], c["wl"], tag, bad, gf="e5m2")
    assert not bad, bad


def test_mxfp8_backward_stages_e5m2_gradients(case):
    """The two backward stage calls with E5M2 gradient operands against the
    oracle's stage functions with grad_fmt="e5m2" on the same given inputs."""
    c, ref, R, I = case, case["ref"], case["p"]["R"], case["wl"].I
    g32 = ref["g"].astype(np.float32)
    u32 = ref["u"].astype(np.float32)
    gu = np.ascontiguousarray(np.concatenate([g32, u32], axis=1))
    out = moe.mxfp8_mlp_bwd_down(to_dev(c["dy"]), to_dev(gu), c["offs"],
                                 c["st"], c["mw"], grad_format="e5m2")
    moe.debug_sync()
    sref = orc.mxfp8_backward_down(c["dy"], g32, u32, c["s"].astype(np.float64),
                                   c["p"]["offsets"], c["inp"]["w_down"],
                                   grad_fmt="e5m2")
    bad = []
    n = c["name"] + " e5m2"
    _check(to_f64(out["dgu"][:R, :I]), sref["dg"], f"{n} stage dg", bad)
    _check(to_f64(out["dgu"][:R, I:]), sref["du"], f"{n} stage du", bad)
    _check(_ds(out["ds"], R), sref["ds"], f"{n} stage ds", bad, "f32")
    for e in range(c["wl"].n_local):
        _check(to_f64(out["dw_down"][e]), sref["dw_down"][e], f"{n} stage dw_down[{e}]", bad)
    ref5 = _ref5(c)
    dgu = np.concatenate([_bits(ref5["dg"]), _bits(ref5["du"])], axis=1)
    out2 = moe.mxfp8_mlp_bwd_gate_up(to_dev(dgu), to_dev(c["x_perm"]), c["offs"],
                                     c["mw"], grad_format="e5m2")
    moe.debug_sync()
    sref2 = orc.mxfp8_mlp_step(c["x_perm"], c["p"]["offsets"], c["s"].astype(np.float64),
                               c["inp"]["w_gate"], c["inp"]["w_up"], c["inp"]["w_down"],
                               c["dy"], bf16_dgu=True, grad_fmt="e5m2")
    _check(to_f64(out2["dx"][:R]), sref2["dx"], f"{n} stage dx", bad)
    for key in ("dw_gate", "dw_up"):
        for e in range(c["wl"].n_local):
            _check(to_f64(out2[key][e]), sref2[key][e], f"{n} stage {key}[{e}]", bad)
    assert not bad, bad
