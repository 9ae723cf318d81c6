"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer outputs (top-k indices, counts, offsets, row_src, inv, x_perm bits)
must match bit for bit; floats must satisfy max|err| <= tau * RMS(ref) with
tau = 2e-2 for bf16 and 1e-4 for fp32 (router logits: 1e-4 in both, as they
accumulate in fp32 from exact inputs).
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_router_amd as moe
import moe_synth as synth
import oracle as orc
from gpu_util import assert_close, print_case, rel_err, to_dev, to_f64

pytestmark = pytest.mark.gpu

SMALL = ["tiny_f32", "c1_tiny_f32", "tiny_bf16", "small_bf16",
         "small_ep_bf16", "mid_bf16"]


def bits(a):
    """Raw bits of a bf16/fp32 tensor or array, for exact comparison."""
    if isinstance(a, torch.Tensor):
        a = a.cpu()
        return (a.view(torch.int16) if a.dtype == torch.bfloat16
                else a.view(torch.int32)).numpy()
    return a.view(np.int16) if a.dtype == np.uint16 else a.view(np.int32)


def _dt(wl):
    return "f32" if wl.dtype == "f32" else "bf16"


def gpu_chain(wl, d, logits=None):
    if wl.router == "gemm":
        idx, w, lg = moe.route_topk(wl.k, x=d["x"], w_router=d["w_router"],
                                    bias=d.get("bias"))
    else:
        idx, w, lg = moe.route_topk(wl.k, logits=d["logits"].clone())
    p = moe.permute(idx, d["x"], wl.e_begin, wl.n_local, topk_w=w, E=wl.E)
    a, y = moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, d["w_gate"],
                           d["w_up"], d["w_down"])
    out = moe.unpermute_combine(y, p.inv)
    moe.debug_sync()
    return dict(idx=idx, w=w, logits=lg, p=p, a=a, y=y, out=out)


@pytest.mark.parametrize("name", SMALL)
def test_small_workload_stepwise(name):
    wl = synth.WORKLOADS[name]
    print_case(name)
    inp = synth.make_inputs(wl)
    ref = orc.moe_layer(wl, inp)
    d = {k: to_dev(v) for k, v in inp.items()}
    g = gpu_chain(wl, d)
    dt = _dt(wl)
    if wl.router == "gemm":
        assert rel_err(to_f64(g["logits"]), ref["logits"]) <= 1e-4
    idx = g["idx"].cpu().numpy()
    np.testing.assert_array_equal(idx, ref["idx"])
    np.testing.assert_allclose(g["w"].cpu().numpy(), ref["topk_w"], atol=2e-6)
    p = g["p"]
    R = ref["R"]
    np.testing.assert_array_equal(p.counts.cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(p.offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(p.row_src.cpu().numpy()[:R], ref["row_src"])
    np.testing.assert_array_equal(p.inv.cpu().numpy(), ref["inv"])
    np.testing.assert_array_equal(bits(p.x_perm[:R]), bits(ref["x_perm"]))
    np.testing.assert_allclose(p.s_perm[:R].cpu().numpy(), ref["s_perm"], atol=2e-6)
    print_case(name, "plain err/RMS a %.2e y %.2e out %.2e" % (
        rel_err(to_f64(g["a"][:R]), ref["a"]), rel_err(to_f64(g["y"][:R]), ref["y"]),
        rel_err(to_f64(g["out"]), ref["out"])))
    assert_close(to_f64(g["a"][:R]), ref["a"], dt, f"{name} a")
    assert_close(to_f64(g["y"][:R]), ref["y"], dt, f"{name} y")
    assert_close(to_f64(g["out"]), ref["out"], dt, f"{name} out")


@pytest.mark.parametrize("name", ["tiny_bf16", "small_bf16", "small_ep_bf16", "mid_bf16"])
def test_gate_up_gather_on_load(name):
    """Reading the token rows through row_src gives the same bits as the
    permuted copy, and the permute without x writes no x_perm."""
    wl = synth.WORKLOADS[name]
    print_case(name, "gather on load")
    inp = synth.make_inputs(wl)
    d = {k: to_dev(v) for k, v in inp.items()}
    g = gpu_chain(wl, d)
    p = g["p"]
    p2 = moe.permute(g["idx"], None, wl.e_begin, wl.n_local, topk_w=g["w"], E=wl.E)
    assert p2.x_perm is None
    a2 = moe.grouped_gate_up_gather(d["x"], p2.row_src, wl.k, p2.offsets,
                                    p2.s_perm, d["w_gate"], d["w_up"])
    moe.debug_sync()
    R = int(p.offsets[-1].item())
    assert torch.equal(p2.offsets, p.offsets)
    np.testing.assert_array_equal(bits(a2[:R]), bits(g["a"][:R]))


def test_topk_bit_exact_on_generated_logits():
    wl = synth.WORKLOADS["c2_ep64_bf16"]
    print_case("topk", wl.name)
    l = synth.make_inputs(wl, with_weights=False)["logits"]
    ridx, rw = orc.topk_softmax(l, wl.k)
    idx, w, _ = moe.route_topk(wl.k, logits=to_dev(l))
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(w.cpu().numpy(), rw, atol=2e-6)
    np.testing.assert_allclose(w.sum(1).cpu().numpy(), 1.0, atol=2e-6)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 6), (100, 7), (256, 8),
                                 (300, 3), (1024, 32)])
def test_topk_ties_and_sizes(E, k):
    print_case("topk sizes", E, k)
    rng = np.random.default_rng(E * 31 + k)
    l = rng.standard_normal((257, E)).astype(np.float32)
    l[0, :] = 0.5                                   # all equal
    l[1, ::3] = l[1].max() + 1.0                    # many equal maxima
    l = np.round(l * 4) / 4                         # plenty of ties
    ridx, rw = orc.topk_softmax(l, k)
    idx, w, _ = moe.route_topk(k, logits=to_dev(l))
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(w.cpu().numpy(), rw, atol=2e-6)


def _edge_inputs(counts, n_local, e_begin, E, k, H, I, seed=7):
    """A routing that gives local experts exactly `counts` slots."""
    rng = np.random.default_rng(seed)
    T = max(max(counts), int(np.ceil(sum(counts) / k))) + 5
    idx = np.full((T, k), -1, dtype=np.int32)
    slots = []
    for e, c in enumerate(counts):
        slots += [e_begin + e] * c
    rng.shuffle(slots)
    # fill token by token, never the same expert twice in a token
    pool = list(slots)
    t = 0
    while pool:
        assert t < T
        row = []
        rest = []
        for s in pool:
            (rest if s in row or len(row) == k else row).append(s)
        idx[t, :len(row)] = row
        pool = rest
        t += 1
    nonlocal_experts = [e for e in range(E) if not (e_begin <= e < e_begin + n_local)]
    for tt in range(T):
        for j in range(k):
            if idx[tt, j] < 0:
                used = set(idx[tt].tolist())
                cand = [e for e in nonlocal_experts if e not in used]
                idx[tt, j] = cand[rng.integers(len(cand))]
    w = rng.random((T, k)); w /= w.sum(1, keepdims=True)
    x = synth.normal_bf16(seed, 1, 0, T * H, 0.0, 1.0).reshape(T, H)
    wg = synth.normal_bf16(seed, 10, 0, n_local * I * H, 0.0, 0.05).reshape(n_local, I, H)
    wu = synth.normal_bf16(seed, 11, 0, n_local * I * H, 0.0, 0.05).reshape(n_local, I, H)
    wd = synth.normal_bf16(seed, 12, 0, n_local * H * I, 0.0, 0.05).reshape(n_local, H, I)
    return idx, w, x, wg, wu, wd


@pytest.mark.parametrize("counts,e_begin,H,I", [
    ([0, 1, 129, 256], 0, 320, 192),     # empty expert, tile straddles, N tails
    ([31, 32, 33, 0, 0, 97], 5, 256, 320),
    ([300], 2, 128, 64),                 # one expert, three m-tiles
])
def test_ffn_edge_segments(counts, e_begin, H, I):
    print_case("edge", counts, e_begin, H, I)
    n_local, E, k = len(counts), 16, 4
    idx, w, x, wg, wu, wd = _edge_inputs(counts, n_local, e_begin, E, k, H, I)
    p_ref = orc.permute(idx, e_begin, n_local)
    np.testing.assert_array_equal(p_ref["counts"], counts)
    xp = orc.gather_rows(x, p_ref["row_src"], k)
    s = w.reshape(-1)[p_ref["row_src"]]
    ex = np.repeat(np.arange(n_local, dtype=np.int32), p_ref["counts"])
    a_ref, y_ref = orc.expert_ffn_rows(xp, ex, s, wg, wu, wd)
    out_ref = orc.combine(y_ref, p_ref["inv"])

    wt = to_dev(w.astype(np.float32))
    p = moe.permute(to_dev(idx), to_dev(x), e_begin, n_local, topk_w=wt, E=E)
    a, y = moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, to_dev(wg),
                           to_dev(wu), to_dev(wd))
    out = moe.unpermute_combine(y, p.inv)
    moe.debug_sync()
    R = p_ref["R"]
    np.testing.assert_array_equal(p.offsets.cpu().numpy(), p_ref["offsets"])
    np.testing.assert_array_equal(p.row_src.cpu().numpy()[:R], p_ref["row_src"])
    np.testing.assert_array_equal(p.inv.cpu().numpy(), p_ref["inv"])
    assert_close(to_f64(a[:R]), a_ref, "bf16", "a")
    assert_close(to_f64(y[:R]), y_ref, "bf16", "y")
    o = to_f64(out)
    assert_close(o, out_ref, "bf16", "out")
    no_local = (p_ref["inv"] < 0).all(axis=1)
    assert no_local.any() and not o[no_local].any()


def test_scale_in_combine_matches_scale_in_ffn():
    wl = synth.WORKLOADS["small_bf16"]
    print_case("scale placement")
    inp = synth.make_inputs(wl)
    d = {k: to_dev(v) for k, v in inp.items()}
    idx, w, _ = moe.route_topk(wl.k, x=d["x"], w_router=d["w_router"],
                               bias=d["bias"])
    p = moe.permute(idx, d["x"], 0, wl.n_local, topk_w=w, E=wl.E)
    _, y1 = moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, d["w_gate"],
                            d["w_up"], d["w_down"])
    o1 = moe.unpermute_combine(y1, p.inv)
    _, y2 = moe.grouped_ffn(p.x_perm, p.offsets, None, d["w_gate"],
                            d["w_up"], d["w_down"])
    o2 = moe.unpermute_combine(y2, p.inv, topk_w=w)
    moe.debug_sync()
    ref = orc.moe_layer(wl, inp, scale_in_ffn=False)["out"]
    assert_close(to_f64(o1), ref, "bf16", "scale in ffn")
    assert_close(to_f64(o2), ref, "bf16", "scale in combine")


def test_empty_token_batch():
    print_case("T=0")
    dev = "cuda"
    l = torch.empty((0, 8), dtype=torch.float32, device=dev)
    idx, w, _ = moe.route_topk(2, logits=l)
    assert idx.shape == (0, 2)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    p = moe.permute(idx, x, 0, 4, topk_w=w, E=8)
    moe.debug_sync()
    assert p.offsets.cpu().tolist() == [0] * 5
    assert p.counts.cpu().tolist() == [0] * 4
    out = moe.unpermute_combine(torch.empty((1, 64), dtype=torch.bfloat16,
                                            device=dev), p.inv)
    assert out.shape == (0, 64)


def test_bitwise_deterministic():
    wl = synth.WORKLOADS["mid_bf16"]
    print_case("determinism")
    inp = synth.make_inputs(wl)
    d = {k: to_dev(v) for k, v in inp.items()}
    g1 = gpu_chain(wl, d)
    g2 = gpu_chain(wl, d)
    R = int(g1["p"].offsets[-1])
    for key in ("idx", "w", "logits", "out"):
        assert torch.equal(g1[key], g2[key]), key
    for key in ("a", "y"):
        assert torch.equal(g1[key][:R], g2[key][:R]), key
    assert torch.equal(g1["p"].row_src[:R], g2["p"].row_src[:R])


def test_step_captured_in_a_graph_replays_bit_exactly():
    """The whole bf16 step (router GEMM + top-k, permute, gate/up, down,
    combine) captured once in a HIP graph and replayed: every replay, with
    eager work and synchronisation between replays, gives the eager result
    bit for bit (the path launches kernels only, no memsets or host syncs)."""
    wl = synth.WORKLOADS["mid_bf16"]
    print_case("graph capture", wl.name)
    inp = synth.make_inputs(wl)
    d = {k: to_dev(v) for k, v in inp.items()}
    dev = d["x"].device
    T, k, H, I = wl.T, wl.k, wl.H, wl.I
    F = T * k
    logits = torch.empty((T, wl.E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    pout = moe.PermuteOut(T, k, H, wl.n_local, torch.bfloat16, dev)
    a = torch.empty((F, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((F, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = moe.ffn_workspace(F, wl.n_local, H, I, torch.bfloat16, dev)

    def step():
        moe.route_topk(k, logits=logits, x=d["x"], w_router=d["w_router"],
                       bias=d.get("bias"), topk_idx=idx, topk_w=w)
        moe.permute(idx, d["x"], wl.e_begin, wl.n_local, topk_w=w, out=pout, E=wl.E)
        moe.grouped_gate_up(pout.x_perm, pout.offsets, pout.s_perm,
                            d["w_gate"], d["w_up"], a=a, workspace=ws)
        moe.grouped_down(a, pout.offsets, d["w_down"], y=y, workspace=ws)
        moe.unpermute_combine(y, pout.inv, out=out)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    ref_idx = idx.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.zero_()
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), rep
        assert torch.equal(out, ref), rep
        # eager work between the replays
        _ = (d["x"].float() @ d["w_router"].float().T).sum().item()


@pytest.mark.parametrize("name", ["small_bf16", "small_ep_bf16"])
def test_ffn_loop_equals_grouped_bit_for_bit(name):
    """The per-expert loop (one set of launches per expert, host-known
    counts) computes exactly what the grouped call computes.  (Bit equality
    needs the same K split on both sides; with K below 16 steps of 64 there
    is none.  Larger shapes are held to the oracle instead, below.)"""
    wl = synth.WORKLOADS[name]
    print_case("loop vs grouped", name)
    inp = synth.make_inputs(wl)
    d = {k: to_dev(v) for k, v in inp.items()}
    g = gpu_chain(wl, d)
    p = g["p"]
    counts = p.counts.cpu().tolist()
    a2, y2 = moe.grouped_ffn_loop(p.x_perm, p.offsets, counts, p.s_perm,
                                  d["w_gate"], d["w_up"], d["w_down"])
    moe.debug_sync()
    R = int(p.offsets[-1].item())
    assert torch.equal(bits_t(g["a"][:R]), bits_t(a2[:R]))
    assert torch.equal(bits_t(g["y"][:R]), bits_t(y2[:R]))


def bits_t(t):
    return t.view(torch.int16)


def test_ffn_loop_edge_segments():
    counts, e_begin, H, I = [0, 1, 129, 256, 0, 64, 65], 0, 256, 320
    n_local, E, k = len(counts), 16, 4
    print_case("loop edge", counts)
    idx, w, x, wg, wu, wd = _edge_inputs(counts, n_local, e_begin, E, k, H, I)
    wt = to_dev(w.astype(np.float32))
    p = moe.permute(to_dev(idx), to_dev(x), e_begin, n_local, topk_w=wt, E=E)
    a, y = moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, to_dev(wg),
                           to_dev(wu), to_dev(wd))
    a2, y2 = moe.grouped_ffn_loop(p.x_perm, p.offsets, counts, p.s_perm,
                                  to_dev(wg), to_dev(wu), to_dev(wd))
    moe.debug_sync()
    R = sum(counts)
    assert torch.equal(bits_t(a[:R]), bits_t(a2[:R]))
    assert torch.equal(bits_t(y[:R]), bits_t(y2[:R]))


@pytest.mark.parametrize("counts,H,I", [
    # gate/up: 5 m-tiles x 8 n-tiles, K 2048 -> split 4; down: 40 tiles,
    # K 1024 -> split 2; one small-class expert and an empty one beside them
    ([200, 0, 129, 70, 40], 2048, 1024),
    # one expert of 65 rows (wide class; the second row-half of the tile
    # holds a single row): 10 gate/up and 4 down tiles, each split 2 ways
    ([65], 1024, 1280),
])
def test_split_k_segments(counts, H, I):
    """Few wide-class tiles: the plan kernel splits K, the last unit of each
    tile adds the fp32 partials.  Held to the oracle, deterministic from call
    to call, and the per-expert loop (other splits) to the oracle too."""
    print_case("split-K", counts, H, I)
    n_local, E, k, e_begin = len(counts), 16, 4, 0
    idx, w, x, wg, wu, wd = _edge_inputs(counts, n_local, e_begin, E, k, H, I,
                                         seed=9)
    p_ref = orc.permute(idx, e_begin, n_local)
    np.testing.assert_array_equal(p_ref["counts"], counts)
    xp = orc.gather_rows(x, p_ref["row_src"], k)
    s = w.reshape(-1)[p_ref["row_src"]]
    ex = np.repeat(np.arange(n_local, dtype=np.int32), p_ref["counts"])
    a_ref, y_ref = orc.expert_ffn_rows(xp, ex, s, wg, wu, wd)

    wt = to_dev(w.astype(np.float32))
    p = moe.permute(to_dev(idx), to_dev(x), e_begin, n_local, topk_w=wt, E=E)
    dwg, dwu, dwd = to_dev(wg), to_dev(wu), to_dev(wd)
    a, y = moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, dwg, dwu, dwd)
    a2, y2 = moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, dwg, dwu, dwd)
    a3, y3 = moe.grouped_ffn_loop(p.x_perm, p.offsets, counts, p.s_perm,
                                  dwg, dwu, dwd)
    moe.debug_sync()
    R = sum(counts)
    assert_close(to_f64(a[:R]), a_ref, "bf16", "a")
    assert_close(to_f64(y[:R]), y_ref, "bf16", "y")
    assert torch.equal(bits_t(a[:R]), bits_t(a2[:R]))
    assert torch.equal(bits_t(y[:R]), bits_t(y2[:R]))
    assert_close(to_f64(a3[:R]), a_ref, "bf16", "loop a")
    assert_close(to_f64(y3[:R]), y_ref, "bf16", "loop y")


def test_ffn_loop_mid_workload_matches_oracle():
    wl = synth.WORKLOADS["mid_bf16"]
    print_case("loop vs oracle", wl.name)
    inp = synth.make_inputs(wl)
    d = {k: to_dev(v) for k, v in inp.items()}
    g = gpu_chain(wl, d)
    p = g["p"]
    counts = p.counts.cpu().tolist()
    a2, y2 = moe.grouped_ffn_loop(p.x_perm, p.offsets, counts, p.s_perm,
                                  d["w_gate"], d["w_up"], d["w_down"])
    moe.debug_sync()
    ref = orc.moe_layer(wl, inp)
    R = int(p.offsets[-1].item())
    assert_close(to_f64(a2[:R]), ref["a"], "bf16", "loop a")
    assert_close(to_f64(y2[:R]), ref["y"], "bf16", "loop y")


@pytest.mark.parametrize("counts,H,I", [
    # split K in both GEMMs (gate/up 4 ways, down 2) beside a small-class
    # expert and an empty one
    ([200, 0, 129, 70, 40], 2048, 1024),
    # gate/up split, down (K 512: too short to split) not
    ([300, 17], 1024, 512),
    # small class only: no split, no claim
    ([1, 64, 33, 0, 7], 512, 384),
])
def test_ffn_one_plan_equals_separate_calls(counts, H, I):
    """moe_grouped_ffn plans both GEMMs in one kernel; its a and y are the
    bits of moe_grouped_gate_up followed by moe_grouped_down (same splits,
    the split counters reset by the gate/up launch for the down launch), and
    moe_grouped_ffn_gather's are those of the gathering gate/up call followed
    by the down call.  Two calls in a row, on one workspace."""
    print_case("one-plan FFN", counts, H, I)
    n_local, E, k, e_begin = len(counts), 16, 4, 0
    idx, w, x, wg, wu, wd = _edge_inputs(counts, n_local, e_begin, E, k, H, I,
                                         seed=11)
    wt = to_dev(w.astype(np.float32))
    dx = to_dev(x)
    p = moe.permute(to_dev(idx), dx, e_begin, n_local, topk_w=wt, E=E)
    dwg, dwu, dwd = to_dev(wg), to_dev(wu), to_dev(wd)
    R_cap, I_ = p.x_perm.shape[0], wg.shape[1]
    ws = moe.ffn_workspace(R_cap, n_local, H, I_, torch.bfloat16, "cuda")
    a1 = moe.grouped_gate_up(p.x_perm, p.offsets, p.s_perm, dwg, dwu,
                             workspace=ws)
    y1 = moe.grouped_down(a1, p.offsets, dwd, workspace=ws)
    a1g = moe.grouped_gate_up_gather(dx, p.row_src, k, p.offsets, p.s_perm,
                                     dwg, dwu, workspace=ws)
    y1g = moe.grouped_down(a1g, p.offsets, dwd, workspace=ws)
    outs = []
    for _ in range(2):
        a, y = moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, dwg, dwu, dwd,
                               workspace=ws)
        ag, yg = moe.grouped_ffn_gather(dx, p.row_src, k, p.offsets, p.s_perm,
                                        dwg, dwu, dwd, workspace=ws)
        outs.append((a, y, ag, yg))
    moe.debug_sync()
    assert moe.read_device_error(ws) == 0
    R = sum(counts)
    for a, y, ag, yg in outs:
        assert torch.equal(bits_t(a[:R]), bits_t(a1[:R]))
        assert torch.equal(bits_t(y[:R]), bits_t(y1[:R]))
        assert torch.equal(bits_t(ag[:R]), bits_t(a1g[:R]))
        assert torch.equal(bits_t(yg[:R]), bits_t(y1g[:R]))


def test_many_small_tiles_per_workgroup_equal_loop():
    """Experts of at most 64 rows and more small-class tiles than
    workgroups: each persistent workgroup walks 2-3 tiles of different
    experts.  The per-expert loop runs every tile on a workgroup of its own;
    each tile's K order (its start rotated by its n-tile) is the same in
    both, so a and y must be the same bits, with x_perm and with rows
    gathered on load.  One expert checked against the oracle too."""
    rng = np.random.default_rng(21)
    counts = [int(c) for c in rng.integers(1, 65, size=80)]
    counts[3], counts[7], counts[11] = 64, 1, 0
    H, I = 2048, 1024
    print_case("small tiles per workgroup", len(counts), "experts", sum(counts), "rows")
    n_local, E, k, e_begin = len(counts), 96, 4, 0
    idx, w, x, wg, wu, wd = _edge_inputs(counts, n_local, e_begin, E, k, H, I,
                                         seed=13)
    wt = to_dev(w.astype(np.float32))
    dx = to_dev(x)
    p = moe.permute(to_dev(idx), dx, e_begin, n_local, topk_w=wt, E=E)
    dwg, dwu, dwd = to_dev(wg), to_dev(wu), to_dev(wd)
    a, y = moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, dwg, dwu, dwd)
    ag, yg = moe.grouped_ffn_gather(dx, p.row_src, k, p.offsets, p.s_perm,
                                    dwg, dwu, dwd)
    a2, y2 = moe.grouped_ffn_loop(p.x_perm, p.offsets, counts, p.s_perm,
                                  dwg, dwu, dwd)
    moe.debug_sync()
    R = sum(counts)
    for got_a, got_y in ((a, y), (ag, yg)):
        assert torch.equal(bits_t(got_a[:R]), bits_t(a2[:R]))
        assert torch.equal(bits_t(got_y[:R]), bits_t(y2[:R]))
    # expert 3 (64 rows) against the oracle
    p_ref = orc.permute(idx, e_begin, n_local)
    b0, b1 = int(p_ref["offsets"][3]), int(p_ref["offsets"][4])
    xp = orc.gather_rows(x, p_ref["row_src"][b0:b1], k)
    s = w.reshape(-1)[p_ref["row_src"][b0:b1]]
    ex = np.zeros(b1 - b0, dtype=np.int32)
    a_ref, y_ref = orc.expert_ffn_rows(xp, ex, s, wg[3:4], wu[3:4], wd[3:4])
    assert_close(to_f64(a[b0:b1]), a_ref, "bf16", "a expert 3")
    assert_close(to_f64(y[b0:b1]), y_ref, "bf16", "y expert 3")
