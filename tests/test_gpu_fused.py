"""The fused decode FFN (moe_grouped_ffn_fused: gate/up, ScaledSwiGLU and
down in one persistent launch on the grouped GEMM's tiles) through the C
ABI, against the oracle.

- Small workloads: a and y per row against the oracle (bf16 rule), with the
  rows read from x_perm and gathered from the token rows (identical bits),
  and repeated calls bit-identical (fixed reduction order, split-K
  included).
- Edge segments: empty experts, one-row experts, experts with more than 64
  rows (several row groups), H not a multiple of the 128-column down unit,
  I of three 64-column gate/up units.
- Full-size EP shares (C2: 4 experts of 116-229 rows, C3: 32 experts of 7-34
  rows, C3 read literally: 32 experts of ~128 rows): every row and token
  against the oracle, and a and y bit for bit against the two grouped
  launches (the same tiles and, at these sizes, the same K splits).
- Segments past R_cap: cut there, memory past R_cap untouched, error word.
- Captured in a HIP graph with the permute and the combine: every replay
  equals the eager result bit for bit (the plan kernel resets the unit
  counters on the device, no memset).
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_router_amd as moe
import moe_synth as synth
import oracle as orc
from gpu_util import assert_close, print_case, rel_err, to_dev, to_f64
from test_gpu_parity import _edge_inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().view(torch.int16).numpy()


@pytest.mark.parametrize("name", ["tiny_bf16", "small_bf16", "small_ep_bf16",
                                  "mid_bf16"])
def test_fused_small_workloads(name):
    wl = synth.WORKLOADS[name]
    print_case(name, "fused")
    inp = synth.make_inputs(wl)
    ref = orc.moe_layer(wl, inp)
    d = {k: to_dev(v) for k, v in inp.items()}
    idx, w, _ = moe.route_topk(wl.k, logits=to_dev(ref["logits"].astype(np.float32)))
    p = moe.permute(idx, d["x"], wl.e_begin, wl.n_local, topk_w=w, E=wl.E)
    a, y = moe.grouped_ffn_fused(p.x_perm, p.offsets, p.s_perm, d["w_gate"],
                                 d["w_up"], d["w_down"])
    a2, y2 = moe.grouped_ffn_fused(d["x"], p.offsets, p.s_perm, d["w_gate"],
                                   d["w_up"], d["w_down"], row_src=p.row_src,
                                   k=wl.k)
    a3, y3 = moe.grouped_ffn_fused(d["x"], p.offsets, p.s_perm, d["w_gate"],
                                   d["w_up"], d["w_down"], row_src=p.row_src,
                                   k=wl.k)
    out = moe.unpermute_combine(y, p.inv)
    moe.debug_sync()
    R = ref["R"]
    np.testing.assert_array_equal(p.offsets.cpu().numpy(), ref["offsets"])
    print_case(name, "fused err/RMS a %.2e y %.2e" % (
        rel_err(to_f64(a[:R]), ref["a"]), rel_err(to_f64(y[:R]), ref["y"])))
    assert_close(to_f64(a[:R]), ref["a"], "bf16", f"{name} a")
    assert_close(to_f64(y[:R]), ref["y"], "bf16", f"{name} y")
    assert_close(to_f64(out), ref["out"], "bf16", f"{name} out")
    np.testing.assert_array_equal(_bits(a2[:R]), _bits(a[:R]))
    np.testing.assert_array_equal(_bits(y2[:R]), _bits(y[:R]))
    np.testing.assert_array_equal(_bits(a3[:R]), _bits(a2[:R]))
    np.testing.assert_array_equal(_bits(y3[:R]), _bits(y2[:R]))


@pytest.mark.parametrize("counts,e_begin,H,I", [
    ([0, 1, 129, 256], 0, 320, 192),     # empty, one row, 3 and 4 row groups
    ([31, 32, 33, 0, 0, 97], 5, 256, 320),
    ([7, 64, 65, 16, 17], 1, 448, 128),  # row-group and 16-row block edges
])
def test_fused_edge_segments(counts, e_begin, H, I):
    print_case("fused edge", counts, e_begin, H, I)
    n_local, E, k = len(counts), 16, 4
    idx, w, x, wg, wu, wd = _edge_inputs(counts, n_local, e_begin, E, k, H, I)
    p_ref = orc.permute(idx, e_begin, n_local)
    np.testing.assert_array_equal(p_ref["counts"], counts)
    xp = orc.gather_rows(x, p_ref["row_src"], k)
    s = w.reshape(-1)[p_ref["row_src"]]
    ex = np.repeat(np.arange(n_local, dtype=np.int32), p_ref["counts"])
    a_ref, y_ref = orc.expert_ffn_rows(xp, ex, s, wg, wu, wd)
    wt = to_dev(w.astype(np.float32))
    p = moe.permute(to_dev(idx), None, e_begin, n_local, topk_w=wt, E=E)
    xd = to_dev(x)
    ws = moe.ffn_workspace(p.row_src.shape[0], n_local, H, I, torch.bfloat16,
                           xd.device)
    a, y = moe.grouped_ffn_fused(xd, p.offsets, p.s_perm, to_dev(wg), to_dev(wu),
                                 to_dev(wd), row_src=p.row_src, k=k, workspace=ws)
    assert moe.read_device_error(ws) == 0
    R = p_ref["R"]
    assert_close(to_f64(a[:R]), a_ref, "bf16", "a")
    assert_close(to_f64(y[:R]), y_ref, "bf16", "y")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["c2_ep64_bf16", "c3_ep8_bf16",
                                  "c3_literal_ep8_bf16"])
def test_fused_ep_share_full(name):
    wl = synth.WORKLOADS[name]
    print_case(name, "fused")
    inp = synth.make_inputs(wl)
    ref = orc.moe_layer(wl, inp)
    d = {k: to_dev(v) for k, v in inp.items()}
    idx, w, _ = moe.route_topk(wl.k, logits=d["logits"].clone())
    p = moe.permute(idx, None, wl.e_begin, wl.n_local, topk_w=w, E=wl.E)
    ws = moe.ffn_workspace(p.row_src.shape[0], wl.n_local, wl.H, wl.I,
                           torch.bfloat16, d["x"].device)
    a, y = moe.grouped_ffn_fused(d["x"], p.offsets, p.s_perm, d["w_gate"],
                                 d["w_up"], d["w_down"], row_src=p.row_src,
                                 k=wl.k, workspace=ws)
    out = moe.unpermute_combine(y, p.inv)
    assert moe.read_device_error(ws) == 0
    moe.debug_sync()
    R = ref["R"]
    o = to_f64(out)
    touched = (ref["inv"] >= 0).any(axis=1)
    assert not o[~touched].any()
    print_case(name, "fused err/RMS a %.2e y %.2e out %.2e" % (
        rel_err(to_f64(a[:R]), ref["a"]), rel_err(to_f64(y[:R]), ref["y"]),
        rel_err(o[touched], ref["out"][touched])))
    assert_close(to_f64(a[:R]), ref["a"], "bf16", f"{name} a")
    assert_close(to_f64(y[:R]), ref["y"], "bf16", f"{name} y")
    assert_close(o[touched], ref["out"][touched], "bf16", f"{name} out")
    # the grouped launches on the same rows: same tiles, same splits
    a2 = moe.grouped_gate_up_gather(d["x"], p.row_src, wl.k, p.offsets,
                                    p.s_perm, d["w_gate"], d["w_up"],
                                    workspace=ws)
    y2 = moe.grouped_down(a2, p.offsets, d["w_down"], workspace=ws)
    moe.debug_sync()
    np.testing.assert_array_equal(_bits(a[:R]), _bits(a2[:R]))
    np.testing.assert_array_equal(_bits(y[:R]), _bits(y2[:R]))


@pytest.mark.parametrize("offsets,R_cap", [
    ([0, 40, 100, 170], 130),          # last segment runs past R_cap
    ([0, 90, 60, 120], 120),           # a decreasing pair
])
def test_fused_rows_past_capacity(offsets, R_cap):
    print_case("fused past R_cap", offsets, R_cap)
    rng = np.random.default_rng(5)
    H, I, n_local, guard = 192, 128, 3, 16
    xp = synth.normal_bf16(5, 1, 0, R_cap * H, 0.0, 1.0).reshape(R_cap, H)
    s = rng.random(R_cap).astype(np.float32)
    wg = synth.normal_bf16(5, 2, 0, n_local * I * H, 0.0, 0.05).reshape(n_local, I, H)
    wu = synth.normal_bf16(5, 3, 0, n_local * I * H, 0.0, 0.05).reshape(n_local, I, H)
    wd = synth.normal_bf16(5, 4, 0, n_local * H * I, 0.0, 0.05).reshape(n_local, H, I)
    dev = torch.device("cuda")
    sentinel = 3.0
    a_full = torch.full((R_cap + guard, I), sentinel, dtype=torch.bfloat16, device=dev)
    y_full = torch.full((R_cap + guard, H), sentinel, dtype=torch.bfloat16, device=dev)
    ws = moe.ffn_workspace(R_cap, n_local, H, I, torch.bfloat16, dev)
    off = np.array(offsets, dtype=np.int32)
    moe.grouped_ffn_fused(to_dev(xp), to_dev(off), to_dev(s), to_dev(wg), to_dev(wu),
                          to_dev(wd), a=a_full[:R_cap], y=y_full[:R_cap],
                          workspace=ws)
    assert moe.read_device_error(ws) == moe.DEVERR_ROWS
    assert (a_full[R_cap:].float() == sentinel).all()
    assert (y_full[R_cap:].float() == sentinel).all()
    # rows owned by exactly one cut segment match the oracle
    owners = np.zeros(R_cap, dtype=int)
    ex = np.full(R_cap, -1)
    for e in range(n_local):
        b = min(max(off[e], 0), R_cap)
        en = min(max(off[e + 1], b), R_cap)
        owners[b:en] += 1
        ex[b:en] = e
    keep = owners == 1
    a_ref, y_ref = orc.expert_ffn_rows(xp[keep], ex[keep], s[keep].astype(np.float64),
                                       wg, wu, wd)
    assert_close(to_f64(a_full[:R_cap])[keep], a_ref, "bf16", "a")
    assert_close(to_f64(y_full[:R_cap])[keep], y_ref, "bf16", "y")
    # a valid call on the same workspace clears the word
    good = np.minimum(off, R_cap)
    good = np.maximum.accumulate(good).astype(np.int32)
    moe.grouped_ffn_fused(to_dev(xp), to_dev(good), to_dev(s), to_dev(wg), to_dev(wu),
                          to_dev(wd), a=a_full[:R_cap], y=y_full[:R_cap],
                          workspace=ws)
    assert moe.read_device_error(ws) == 0


def test_fused_step_in_a_graph_replays_bit_exactly():
    wl = synth.WORKLOADS["c3_ep8_bf16"]
    print_case("fused graph capture", wl.name)
    inp = synth.make_inputs(wl)
    d = {k: to_dev(v) for k, v in inp.items()}
    dev = d["x"].device
    T, k, H, I = wl.T, wl.k, wl.H, wl.I
    F = T * k
    pout = moe.PermuteOut(T, k, H, wl.n_local, torch.bfloat16, dev, with_x=False)
    a = torch.empty((F, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((F, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = moe.ffn_workspace(F, wl.n_local, H, I, torch.bfloat16, dev)
    idx, w, _ = moe.route_topk(k, logits=d["logits"].clone())

    def step():
        moe.permute(idx, None, wl.e_begin, wl.n_local, topk_w=w, out=pout, E=wl.E)
        moe.grouped_ffn_fused(d["x"], pout.offsets, pout.s_perm, d["w_gate"],
                              d["w_up"], d["w_down"], row_src=pout.row_src, k=k,
                              a=a, y=y, workspace=ws)
        moe.unpermute_combine(y, pout.inv, out=out)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        _ = (d["x"].float().sum()).item()
