"""MXFP8 path through the C ABI against the CPU oracle.

Codes and scales of given bf16 inputs must match bit for bit.  Float
outputs must meet max(|err| - bf16 slack) <= 6e-2 * RMS of each row of the
reference (the oracle dequantises exactly and works in fp64).

Tensors handed from one operation to the next are bf16 and are quantised
again by the next GEMM.  When such a tensor is computed on both sides (fp32
on the device, fp64 in the oracle), a value near an E4M3 rounding boundary
can be quantised to neighbouring codes on the two sides; each code choice is
correct for its input.  So every GEMM stage is checked on the oracle's own
bf16 hand-off tensors, where both sides quantise identical values, and the
fused calls are checked end to end on what no such decision feeds (g, u, a,
ds) plus an aggregate bound on the rest.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_router_amd as moe
import moe_synth as synth
import oracle as orc
from gpu_util import print_case, rel_err, scaled_excess, to_dev, to_f64

pytestmark = pytest.mark.gpu
TAU = 6e-2


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
    """bf16 bits of values the oracle already rounded to bf16 (exact)."""
    v = orc.round_bf16(v)
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _check(got, ref, what, bad):
    e = scaled_excess(got, ref, "bf16")
    print_case(what, f"row excess {e:.2e}, plain {rel_err(got, ref):.2e}")
    if not e <= TAU:
        bad.append(f"{what}: {e:.3e}")


def _frob(got, ref, what, bad, bound=2e-2):
    r = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print_case(what, f"relative Frobenius error {r:.2e}")
    if not r <= bound:
        bad.append(f"{what}: frobenius {r:.3e}")


@pytest.fixture(scope="module", params=["small_mxfp8", "mid_mxfp8"])
def case(request):
    name = request.param
    print_case(name)
    wl, inp, p, x_perm, s, dy, ref = _mx_case(name)
    d = {k: to_dev(inp[k]) for k in ("w_gate", "w_up", "w_down")}
    mw = moe.MxWeights(d["w_gate"], d["w_up"], d["w_down"])
    return dict(name=name, wl=wl, p=p, x_perm=x_perm, s=s, dy=dy, ref=ref,
                mw=mw, offs=to_dev(p["offsets"]), st=to_dev(s))


def test_mxfp8_down_projection_stage(case):
    """y = MX(a) MX(W_d)^T on the oracle's bf16 a."""
    c, ref, R = case, case["ref"], case["p"]["R"]
    y = moe.grouped_linear_mxfp8(to_dev(_bits(ref["a"])), c["offs"],
                                 c["wl"].n_local, c["mw"].wd, c["mw"].wds)
    moe.debug_sync()
    bad = []
    _check(to_f64(y[:R]), ref["y"], f"{c['name']} stage y", bad)
    assert not bad, bad


def test_mxfp8_backward_down_stage(case):
    """da -> SwiGLU backward -> dg, du, ds, and dW_down, on the oracle's
    bf16 a, g, u."""
    c, ref, R, I = case, case["ref"], case["p"]["R"], case["wl"].I
    gu = np.concatenate([_bits(ref["g"]), _bits(ref["u"])], axis=1)
    out = moe.mxfp8_mlp_bwd_down(to_dev(c["dy"]), to_dev(_bits(ref["a"])),
                                 to_dev(gu), c["offs"], c["st"], c["mw"])
    moe.debug_sync()
    bad = []
    n = c["name"]
    _check(to_f64(out["dgu"][:R, :I]), ref["dg"], f"{n} stage dg", bad)
    _check(to_f64(out["dgu"][:R, I:]), ref["du"], f"{n} stage du", bad)
    _check(out["ds"][:R].cpu().numpy().astype(np.float64), ref["ds"],
           f"{n} stage ds", bad)
    for e in range(c["wl"].n_local):
        _check(to_f64(out["dw_down"][e]), ref["dw_down"][e],
               f"{n} stage dw_down[{e}]", bad)
    assert not bad, bad


def test_mxfp8_backward_gate_up_stage(case):
    """dX, dW_gate, dW_up on the oracle's bf16 dg, du."""
    c, ref, R = case, case["ref"], case["p"]["R"]
    dgu = np.concatenate([_bits(ref["dg"]), _bits(ref["du"])], axis=1)
    out = moe.mxfp8_mlp_bwd_gate_up(to_dev(dgu), to_dev(c["x_perm"]),
                                    c["offs"], c["mw"])
    moe.debug_sync()
    bad = []
    n = c["name"]
    _check(to_f64(out["dx"][:R]), ref["dx"], f"{n} stage dx", bad)
    for key in ("dw_gate", "dw_up"):
        for e in range(c["wl"].n_local):
            _check(to_f64(out[key][e]), ref[key][e], f"{n} stage {key}[{e}]", bad)
    assert not bad, bad


def test_mxfp8_fused_quantisation_equals_separate(case):
    """The SwiGLU epilogue quantises a (forward) and [dg | du] (backward) from
    the bf16 values it stores; the fused calls must therefore equal the
    stage calls, which quantise the stored bf16 tensors with the row
    quantiser (pinned to the oracle bit for bit, every bf16 value at every
    scale), bit for bit: y against the grouped linear on the returned a and
    against the two-call forward (gate/up, then the down projection from the
    workspace codes), and dX, dW against the two backward stages."""
    c, R = case, case["p"]["R"]
    wl = c["wl"]
    xt = to_dev(c["x_perm"])
    xq, xs = moe.mxfp8_quantize(xt, 0)
    a, gu, y = moe.mxfp8_mlp_fwd(xq, xs, c["offs"], c["st"], c["mw"])
    y_sep = moe.grouped_linear_mxfp8(a, c["offs"], wl.n_local, c["mw"].wd, c["mw"].wds)
    R_cap = xq.shape[0]
    nb = moe.lib().moe_grouped_mlp_mxfp8_fwd_workspace_bytes(R_cap, wl.n_local, wl.H, wl.I)
    ws = torch.empty(nb, dtype=torch.uint8, device=xq.device)
    moe.mxfp8_mlp_fwd(xq, xs, c["offs"], c["st"], c["mw"], workspace=ws, down=False)
    y_two = moe.mxfp8_mlp_fwd_down(c["offs"], c["mw"], ws, R_cap)
    dy = to_dev(c["dy"])
    g = moe.mxfp8_mlp_bwd(dy, xt, a, gu, c["offs"], c["st"], c["mw"])
    d1 = moe.mxfp8_mlp_bwd_down(dy, a, gu, c["offs"], c["st"], c["mw"])
    d2 = moe.mxfp8_mlp_bwd_gate_up(d1["dgu"], xt, c["offs"], c["mw"])
    moe.debug_sync()
    print_case(c["name"], "fused vs stage calls, rows", R)
    assert torch.equal(y[:R], y_sep[:R])
    assert torch.equal(y[:R], y_two[:R])
    assert torch.equal(g["ds"][:R], d1["ds"][:R])
    assert torch.equal(g["dw_down"], d1["dw_down"])
    assert torch.equal(g["dx"][:R], d2["dx"][:R])
    assert torch.equal(g["dw_gate"], d2["dw_gate"])
    assert torch.equal(g["dw_up"], d2["dw_up"])


def test_mxfp8_fused_forward_backward(case):
    c, ref, R, I = case, case["ref"], case["p"]["R"], case["wl"].I
    xt = to_dev(c["x_perm"])
    xq, xs = moe.mxfp8_quantize(xt, 0)
    a, gu, y = moe.mxfp8_mlp_fwd(xq, xs, c["offs"], c["st"], c["mw"])
    g = moe.mxfp8_mlp_bwd(to_dev(c["dy"]), xt, a, gu, c["offs"], c["st"],
                          c["mw"])
    moe.debug_sync()
    bad = []
    n = c["name"]
    _check(to_f64(gu[:R, :I]), ref["g"], f"{n} g", bad)
    _check(to_f64(gu[:R, I:]), ref["u"], f"{n} u", bad)
    _check(to_f64(a[:R]), ref["a"], f"{n} a", bad)
    _check(g["ds"][:R].cpu().numpy().astype(np.float64), ref["ds"], f"{n} ds", bad)
    _frob(to_f64(y[:R]), ref["y"], f"{n} y", bad)
    _frob(to_f64(g["dx"][:R]), ref["dx"], f"{n} dx", bad)
    for key in ("dw_gate", "dw_up", "dw_down"):
        _frob(to_f64(g[key]), ref[key], f"{n} {key}", bad)
    assert not bad, bad


def test_mxfp8_experts_without_rows():
    """Experts 0 and 2 of four receive no rows: their weight-gradient GEMMs
    run over empty K ranges and must return exact zeros, and the fused calls
    must still equal the stage calls bit for bit."""
    wl = synth.WORKLOADS["small_mxfp8"]
    R = 300
    inp = synth.make_inputs(wl, tokens=R)
    offsets = np.array([0, 0, 127, 127, R], np.int32)
    x_perm = inp["x"]
    s = np.random.default_rng(11).uniform(0.05, 1.0, R).astype(np.float32)
    dy = synth.make_dy(wl, R)
    ref = orc.mxfp8_mlp_step(x_perm, offsets, s.astype(np.float64),
                             inp["w_gate"], inp["w_up"], inp["w_down"], dy)
    d = {k: to_dev(inp[k]) for k in ("w_gate", "w_up", "w_down")}
    mw = moe.MxWeights(d["w_gate"], d["w_up"], d["w_down"])
    offs, st, xt, dyt = to_dev(offsets), to_dev(s), to_dev(x_perm), to_dev(dy)
    print_case("small_mxfp8 experts 0, 2 empty", "rows", R)
    xq, xs = moe.mxfp8_quantize(xt, 0)
    a, gu, y = moe.mxfp8_mlp_fwd(xq, xs, offs, st, mw)
    g = moe.mxfp8_mlp_bwd(dyt, xt, a, gu, offs, st, mw)
    d1 = moe.mxfp8_mlp_bwd_down(dyt, a, gu, offs, st, mw)
    d2 = moe.mxfp8_mlp_bwd_gate_up(d1["dgu"], xt, offs, mw)
    moe.debug_sync()
    for key in ("dw_gate", "dw_up", "dw_down"):
        for e in (0, 2):
            assert not g[key][e].any(), (key, e)
    assert torch.equal(g["dw_down"], d1["dw_down"])
    assert torch.equal(g["dx"][:R], d2["dx"][:R])
    assert torch.equal(g["dw_gate"], d2["dw_gate"])
    assert torch.equal(g["dw_up"], d2["dw_up"])
    bad = []
    _check(to_f64(a[:R]), ref["a"], "empty-expert a", bad)
    _check(g["ds"][:R].cpu().numpy().astype(np.float64), ref["ds"],
           "empty-expert ds", bad)
    _frob(to_f64(y[:R]), ref["y"], "empty-expert y", bad)
    _frob(to_f64(g["dx"][:R]), ref["dx"], "empty-expert dx", bad)
    for key in ("dw_gate", "dw_up", "dw_down"):
        for e in (1, 3):
            _frob(to_f64(g[key][e]), ref[key][e], f"empty-expert {key}[{e}]", bad)
    assert not bad, bad


def test_mxfp8_tiny_ragged_segments():
    """Segments of 3, 0, 1 and 37 rows at the smallest shapes (H = I = 512):
    every tile is mostly padding and the weight-gradient K ranges are one
    256-row block or empty.  The fused calls equal the stage calls bit for
    bit; a, ds and the aggregate y, dX meet the oracle; the weight gradients
    are checked row by row on the oracle's own bf16 hand-off tensors (with
    one or three rows a segment's MX blocks hold single values, so a code
    decided differently on the two sides would not average out)."""
    wl = synth.WORKLOADS["small_mxfp8"]
    counts = [3, 0, 1, 37]
    R = sum(counts)
    inp = synth.make_inputs(wl, tokens=R)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x_perm = inp["x"]
    s = np.random.default_rng(5).uniform(0.05, 1.0, R).astype(np.float32)
    dy = synth.make_dy(wl, R)
    ref = orc.mxfp8_mlp_step(x_perm, offsets, s.astype(np.float64),
                             inp["w_gate"], inp["w_up"], inp["w_down"], dy)
    d = {k: to_dev(inp[k]) for k in ("w_gate", "w_up", "w_down")}
    mw = moe.MxWeights(d["w_gate"], d["w_up"], d["w_down"])
    offs, st, xt, dyt = to_dev(offsets), to_dev(s), to_dev(x_perm), to_dev(dy)
    print_case("small_mxfp8 segments", counts)
    xq, xs = moe.mxfp8_quantize(xt, 0)
    a, gu, y = moe.mxfp8_mlp_fwd(xq, xs, offs, st, mw)
    g = moe.mxfp8_mlp_bwd(dyt, xt, a, gu, offs, st, mw)
    d1 = moe.mxfp8_mlp_bwd_down(dyt, a, gu, offs, st, mw)
    d2 = moe.mxfp8_mlp_bwd_gate_up(d1["dgu"], xt, offs, mw)
    # the weight gradients on the oracle's hand-off tensors
    gu_ref = np.concatenate([_bits(ref["g"]), _bits(ref["u"])], axis=1)
    h1 = moe.mxfp8_mlp_bwd_down(dyt, to_dev(_bits(ref["a"])), to_dev(gu_ref),
                                offs, st, mw)
    dgu_ref = np.concatenate([_bits(ref["dg"]), _bits(ref["du"])], axis=1)
    h2 = moe.mxfp8_mlp_bwd_gate_up(to_dev(dgu_ref), xt, offs, mw)
    moe.debug_sync()
    for key in ("dw_gate", "dw_up", "dw_down"):
        assert not g[key][1].any(), key
    assert torch.equal(g["dw_down"], d1["dw_down"])
    assert torch.equal(g["dx"][:R], d2["dx"][:R])
    assert torch.equal(g["dw_gate"], d2["dw_gate"])
    assert torch.equal(g["dw_up"], d2["dw_up"])
    bad = []
    _check(to_f64(a[:R]), ref["a"], "tiny a", bad)
    _check(g["ds"][:R].cpu().numpy().astype(np.float64), ref["ds"], "tiny ds", bad)
    _frob(to_f64(y[:R]), ref["y"], "tiny y", bad)
    _frob(to_f64(g["dx"][:R]), ref["dx"], "tiny dx", bad)
    for e in (0, 2, 3):
        _check(to_f64(h1["dw_down"][e]), ref["dw_down"][e], f"tiny dw_down[{e}]", bad)
        _check(to_f64(h2["dw_gate"][e]), ref["dw_gate"][e], f"tiny dw_gate[{e}]", bad)
        _check(to_f64(h2["dw_up"][e]), ref["dw_up"][e], f"tiny dw_up[{e}]", bad)
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
    gu = torch.empty((R_cap, 2 * I), dtype=bf, device=dev)
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
        moe.mxfp8_mlp_bwd(dyt, xt, a, gu, c["offs"], c["st"], c["mw"],
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
