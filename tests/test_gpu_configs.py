"""The full-size workloads through the C ABI, against the oracle.

EP64 share (4 experts) and EP8 share (32 experts, on 512 tokens and on all
4096): every row and token is checked.  Full layer (8192 tokens, 256 experts): the router GEMM and top-k
over all tokens, the permute in full (bit-exact), and the FFN / combine on a
seeded sample of rows and tokens (every expert's first and last row plus 512
random rows; 96 random tokens), which the oracle computes one by one.  The
bf16 forward on the MXFP8 step's shapes (8 experts of about 4096 rows) is
sampled the same way.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_router_amd as moe
import moe_synth as synth
import oracle as orc
from gpu_util import assert_close, print_case, rel_err, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().view(torch.int16).numpy()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["c2_ep64_bf16", "c3_ep8_bf16",
                                  "c3_literal_ep8_bf16"])
def test_ep_share_full(name):
    wl = synth.WORKLOADS[name]
    print_case(name)
    inp = synth.make_inputs(wl)
    ref = orc.moe_layer(wl, inp)
    d = {k: to_dev(v) for k, v in inp.items()}
    idx, w, _ = moe.route_topk(wl.k, logits=d["logits"].clone())
    p = moe.permute(idx, d["x"], wl.e_begin, wl.n_local, topk_w=w, E=wl.E)
    a, y = moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, d["w_gate"],
                           d["w_up"], d["w_down"])
    out = moe.unpermute_combine(y, p.inv)
    moe.debug_sync()
    R = ref["R"]
    print_case(name, "R", R, "counts", ref["counts"].tolist()[:8])
    np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])
    np.testing.assert_array_equal(p.offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(p.row_src.cpu().numpy()[:R], ref["row_src"])
    np.testing.assert_array_equal(p.inv.cpu().numpy(), ref["inv"])
    np.testing.assert_array_equal(_bits(p.x_perm[:R]), ref["x_perm"].view(np.int16))
    o = to_f64(out)
    touched = (ref["inv"] >= 0).any(axis=1)
    # rows of tokens with no local expert are exact zeros; the float check
    # runs over the tokens this GPU computes (RMS over those rows)
    assert not o[~touched].any()
    print_case(name, "plain err/RMS a %.2e y %.2e out %.2e" % (
        rel_err(to_f64(a[:R]), ref["a"]), rel_err(to_f64(y[:R]), ref["y"]),
        rel_err(o[touched], ref["out"][touched])))
    assert_close(to_f64(a[:R]), ref["a"], "bf16", f"{name} a")
    assert_close(to_f64(y[:R]), ref["y"], "bf16", f"{name} y")
    assert_close(o[touched], ref["out"][touched], "bf16", f"{name} out")


@pytest.fixture(scope="module")
def c4():
    wl = synth.WORKLOADS["c4_full_bf16"]
    print_case("c4 generate")
    inp = synth.make_inputs(wl, with_weights=False)
    dev = {k: to_dev(v) for k, v in inp.items()}
    # weights: generated and moved in slices of 32 experts
    wg = torch.empty((wl.n_local, wl.I, wl.H), dtype=torch.bfloat16, device="cuda")
    wu = torch.empty_like(wg)
    wd = torch.empty((wl.n_local, wl.H, wl.I), dtype=torch.bfloat16, device="cuda")
    host = {"w_gate": [], "w_up": [], "w_down": []}
    for e0 in range(0, wl.n_local, 32):
        part = synth.make_weights(wl, range(e0, min(wl.n_local, e0 + 32)))
        for key, dst in (("w_gate", wg), ("w_up", wu), ("w_down", wd)):
            dst[e0:e0 + part[key].shape[0]].copy_(to_dev(part[key]))
            host[key].append(part[key])
    for key in host:
        inp[key] = np.concatenate(host[key])
    dev.update(w_gate=wg, w_up=wu, w_down=wd)
    print_case("c4 oracle routing")
    ridx, rw, l32, l64 = orc.routing_of(wl, inp)
    return wl, inp, dev, dict(idx=ridx, w=rw, l32=l32, l64=l64)


@pytest.mark.timeout(300)
def test_c4_router_and_topk(c4):
    wl, inp, d, r = c4
    print_case("c4 router")
    idx, w, logits = moe.route_topk(wl.k, x=d["x"], w_router=d["w_router"],
                                    bias=d["bias"])
    moe.debug_sync()
    lg = to_f64(logits)
    e = rel_err(lg, r["l64"])
    assert e <= 1e-4, e
    gi = idx.cpu().numpy()
    diff = (gi != r["idx"]).any(axis=1)
    print_case("c4 router", f"logit err/RMS {e:.2e}, tokens with other top-k {diff.sum()}")
    assert diff.sum() <= wl.T // 1000
    # where the choice differs, it must be a near-tie of the fp64 logits
    tol = 8 * e * np.sqrt(np.mean(r["l64"] ** 2))
    for t in np.nonzero(diff)[0]:
        l = r["l64"][t]
        got_min = l[gi[t]].min()
        other = np.setdiff1d(np.arange(wl.E), gi[t])
        assert l[other].max() - got_min <= tol, t


@pytest.mark.timeout(300)
def test_c4_topk_on_oracle_logits_bit_exact(c4):
    """Softmax -> top-8 -> renormalise at the full layer's size (8192 tokens
    over 256 experts) on the oracle's logits rounded to fp32: both sides take
    the choice on the same fp32 values, so the indices match bit for bit."""
    wl, inp, d, r = c4
    print_case("c4 top-k on oracle logits")
    idx, w, _ = moe.route_topk(wl.k, logits=to_dev(r["l32"]))
    moe.debug_sync()
    np.testing.assert_array_equal(idx.cpu().numpy(), r["idx"])
    np.testing.assert_allclose(w.cpu().numpy(), r["w"], atol=2e-6)


@pytest.mark.timeout(300)
def test_c4_permute_ffn_combine_sampled(c4):
    wl, inp, d, r = c4
    print_case("c4 permute/ffn")
    p_ref = orc.permute(r["idx"], 0, wl.n_local)
    R = p_ref["R"]
    assert R == wl.T * wl.k
    w32 = r["w"].astype(np.float32)
    p = moe.permute(to_dev(r["idx"]), d["x"], 0, wl.n_local, topk_w=to_dev(w32), E=wl.E)
    a, y = moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, d["w_gate"],
                           d["w_up"], d["w_down"])
    out = moe.unpermute_combine(y, p.inv)
    moe.debug_sync()
    np.testing.assert_array_equal(p.counts.cpu().numpy(), p_ref["counts"])
    np.testing.assert_array_equal(p.offsets.cpu().numpy(), p_ref["offsets"])
    np.testing.assert_array_equal(p.row_src.cpu().numpy()[:R], p_ref["row_src"])
    np.testing.assert_array_equal(p.inv.cpu().numpy(), p_ref["inv"])
    # x_perm: all rows bit-exact against the token rows
    xp = _bits(p.x_perm[:R])
    np.testing.assert_array_equal(xp, inp["x"].view(np.int16)[p_ref["row_src"] // wl.k])
    print_case("c4 loads min/median/max",
               p_ref["counts"].min(), int(np.median(p_ref["counts"])), p_ref["counts"].max())
    # sampled rows: first and last of each expert + 512 random
    rng = np.random.default_rng(0)
    off = p_ref["offsets"]
    rows = set(rng.choice(R, 512, replace=False).tolist())
    for e in range(wl.n_local):
        if off[e + 1] > off[e]:
            rows.update((int(off[e]), int(off[e + 1]) - 1))
    rows = np.array(sorted(rows))
    ex = (np.searchsorted(off, rows, side="right") - 1).astype(np.int32)
    xs = inp["x"][p_ref["row_src"][rows] // wl.k]
    s = w32.reshape(-1)[p_ref["row_src"][rows]].astype(np.float64)
    a_ref, y_ref = orc.expert_ffn_rows(xs, ex, s, inp["w_gate"], inp["w_up"],
                                       inp["w_down"])
    ea = assert_close(to_f64(a[rows]), a_ref, "bf16", "c4 a")
    ey = assert_close(to_f64(y[rows]), y_ref, "bf16", "c4 y")
    toks = rng.choice(wl.T, 96, replace=False)
    o_ref = orc.moe_tokens(inp["x"], r["idx"], w32.astype(np.float64), toks, 0,
                           wl.n_local, inp["w_gate"], inp["w_up"], inp["w_down"])
    eo = assert_close(to_f64(out[toks]), o_ref, "bf16", "c4 out")
    print_case("c4", f"err/RMS a {ea:.2e} y {ey:.2e} out {eo:.2e}")
    # the gather-on-load gate/up the benchmark times: same bits as on x_perm
    a_g = moe.grouped_gate_up_gather(d["x"], p.row_src, wl.k, p.offsets,
                                     p.s_perm, d["w_gate"], d["w_up"])
    moe.debug_sync()
    assert torch.equal(a_g[:R], a[:R])


@pytest.mark.timeout(300)
def test_c4_end_to_end_sampled(c4):
    wl, inp, d, r = c4
    print_case("c4 end to end")
    idx, w, _ = moe.route_topk(wl.k, x=d["x"], w_router=d["w_router"],
                               bias=d["bias"])
    p = moe.permute(idx, d["x"], 0, wl.n_local, topk_w=w, E=wl.E)
    a, y = moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, d["w_gate"],
                           d["w_up"], d["w_down"])
    out = moe.unpermute_combine(y, p.inv)
    moe.debug_sync()
    same = (idx.cpu().numpy() == r["idx"]).all(axis=1)
    rng = np.random.default_rng(1)
    toks = rng.choice(np.nonzero(same)[0], 64, replace=False)
    o_ref = orc.moe_tokens(inp["x"], r["idx"], r["w"], toks, 0, wl.n_local,
                           inp["w_gate"], inp["w_up"], inp["w_down"])
    assert_close(to_f64(out[toks]), o_ref, "bf16", "c4 end-to-end out")


@pytest.mark.timeout(300)
def test_c5_shape_bf16_sampled():
    """16384 tokens, top-2 of 8 experts, H 4096, I 8192 in bf16: the permute
    in full, a and y on every expert's first and last row plus 256 random
    rows, out on 64 random tokens; the gather-on-load gate/up the benchmark
    times gives the same bits as the one on x_perm."""
    wl = synth.WORKLOADS["c5_shape_bf16"]
    print_case("c5-shape bf16 generate")
    inp = synth.make_inputs(wl)
    d = {k: to_dev(v) for k, v in inp.items()}
    idx, w, _ = moe.route_topk(wl.k, logits=d["logits"].clone())
    ridx, rw = orc.topk_softmax(inp["logits"], wl.k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(w.cpu().numpy() - rw).max() <= 1e-6
    p_ref = orc.permute(ridx, 0, wl.n_local)
    R = p_ref["R"]
    # the FFN scales rows by the oracle's weights (rounded to fp32), so that
    # every expected value below derives from the oracle alone
    w32 = rw.astype(np.float32)
    p = moe.permute(idx, d["x"], 0, wl.n_local, topk_w=to_dev(w32), E=wl.E)
    a, y = moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, d["w_gate"],
                           d["w_up"], d["w_down"])
    out = moe.unpermute_combine(y, p.inv)
    a_g = moe.grouped_gate_up_gather(d["x"], p.row_src, wl.k, p.offsets,
                                     p.s_perm, d["w_gate"], d["w_up"])
    moe.debug_sync()
    np.testing.assert_array_equal(p.offsets.cpu().numpy(), p_ref["offsets"])
    np.testing.assert_array_equal(p.row_src.cpu().numpy()[:R], p_ref["row_src"])
    np.testing.assert_array_equal(p.inv.cpu().numpy(), p_ref["inv"])
    assert torch.equal(a_g[:R], a[:R])
    print_case("c5-shape bf16 rows per expert", p_ref["counts"].tolist())
    rng = np.random.default_rng(2)
    off = p_ref["offsets"]
    rows = set(rng.choice(R, 256, replace=False).tolist())
    for e in range(wl.n_local):
        if off[e + 1] > off[e]:
            rows.update((int(off[e]), int(off[e + 1]) - 1))
    rows = np.array(sorted(rows))
    ex = (np.searchsorted(off, rows, side="right") - 1).astype(np.int32)
    xs = inp["x"][p_ref["row_src"][rows] // wl.k]
    s = w32.reshape(-1)[p_ref["row_src"][rows]].astype(np.float64)
    a_ref, y_ref = orc.expert_ffn_rows(xs, ex, s, inp["w_gate"], inp["w_up"],
                                       inp["w_down"])
    ea = assert_close(to_f64(a[rows]), a_ref, "bf16", "c5-shape a")
    ey = assert_close(to_f64(y[rows]), y_ref, "bf16", "c5-shape y")
    toks = rng.choice(wl.T, 64, replace=False)
    o_ref = orc.moe_tokens(inp["x"], ridx, w32.astype(np.float64), toks, 0,
                           wl.n_local, inp["w_gate"], inp["w_up"], inp["w_down"])
    eo = assert_close(to_f64(out[toks]), o_ref, "bf16", "c5-shape out")
    print_case("c5-shape bf16", f"err/RMS a {ea:.2e} y {ey:.2e} out {eo:.2e}")
