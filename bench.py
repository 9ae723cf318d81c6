"""Benchmark of the MoE expert-layer path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
router GEMM + softmax/top-k, permute, grouped gate/up with the SwiGLU x
routing-scale epilogue (reading the token rows through row_src), grouped
down, combine (default workload: the full layer, 8192 tokens, hidden 7168,
256 experts, top-8, intermediate 2048).  The EP-share workloads (--workload
c2_ep64_bf16 | c3_ep8_bf16) route before the timed region and time permute
+ FFN + combine; --workload c5_mxfp8 times the MXFP8 grouped-MLP training
step.

Prints one JSON line.  `value` is the grouped-FFN (+ router) TFLOP/s of the
whole step with inputs resident in HBM, timed over exactly K steps replayed
from a HIP graph of the step (the same kernels without host launch overhead;
--no-graph times eager launches, and the eager time is reported beside it);
`roofline` is for the dominant kernel (the grouped gate/up GEMM), timed with
HIP events on its stream during K eager steps; `cpu_baseline` is the CPU
oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mixture_experts_expert_router_amd as moe  # noqa: E402
import moe_synth as synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5033.2       # MI355X dense fp8 (MX-scaled) MFMA
METRIC = "grouped MoE FFN TFLOP/s + rows/s per layer; % MFMA peak or % HBM BW"
TIMING_GRAPH = ("K replays of the step captured in a HIP graph (same kernels, no host "
                "launch overhead), after W eager warmup steps and K eager steps timed "
                "with HIP events")
TIMING_EAGER = "K eager steps"


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE passes (profiles/traffic.json), or None
    when there are none or the kernel's sources changed since they were
    taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[workload]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, "mixture_experts_expert_router_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return int(rec["bytes"])


def copy_probe(mb, dev):
    """One elementwise copy of `mb` MiB (read + write) after the timed
    region: the reference for scaling HBM byte counters."""
    n = mb * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"copy probe: {n * 2} bytes read, {n * 2} bytes written")


def to_dev(a, dev):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def make_device_workload(wl, dev, weight_copies):
    """Inputs on the device; host copies kept for the CPU-baseline leg."""
    inp = synth.make_inputs(wl, with_weights=False)
    d = {k: to_dev(v, dev) for k, v in inp.items()}
    host_w = {"w_gate": [], "w_up": [], "w_down": []}
    copies = []
    for c in range(weight_copies):
        wg = torch.empty((wl.n_local, wl.I, wl.H), dtype=torch.bfloat16, device=dev)
        wu = torch.empty_like(wg)
        wd = torch.empty((wl.n_local, wl.H, wl.I), dtype=torch.bfloat16, device=dev)
        copies.append((wg, wu, wd))
    step = 32
    for e0 in range(0, wl.n_local, step):
        e1 = min(wl.n_local, e0 + step)
        part = synth.make_weights(wl, range(wl.e_begin + e0, wl.e_begin + e1))
        for c in copies:
            for dst, key in zip(c, ("w_gate", "w_up", "w_down")):
                dst[e0:e1].copy_(to_dev(part[key], dev))
        for key in host_w:
            host_w[key].append(part[key])
    for key in host_w:
        inp[key] = np.concatenate(host_w[key])
    return inp, d, copies


def algorithmic(wl, R, n_touched, gather=True):
    """FLOPs and HBM bytes of one step: every touched expert's weights once,
    the expert rows of x read once per row (gathered by the gate/up GEMM, or
    read by the permute and written + re-read as x_perm), a and y written and
    read once, out written once."""
    H, I, T, E, k = wl.H, wl.I, wl.T, wl.E, wl.k
    flop_ffn = 6.0 * R * H * I
    flop_router = 2.0 * T * H * E if wl.router == "gemm" else 0.0
    w_bytes = 3.0 * n_touched * H * I * 2
    act = 2.0
    gate_up_bytes = 2.0 * n_touched * H * I * 2 + R * H * act + R * I * act
    x_bytes = R * H * act if gather else T * H * act + 2 * R * H * act
    step_bytes = (w_bytes + x_bytes
                  + 2 * R * I * act                # a write + read
                  + 2 * R * H * act                # y write + read
                  + T * H * act)                   # out write
    if wl.router == "gemm":
        step_bytes += T * H * act + E * H * act + 2 * T * E * 4
    return dict(flop_ffn=flop_ffn, flop_router=flop_router,
                gate_up_flop=4.0 * R * H * I, gate_up_bytes=gate_up_bytes,
                step_bytes=step_bytes)


def capture_steps(step_fns):
    """One HIP graph per callable (each runs one step with preallocated
    buffers), or None when capture is not possible here."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for fn in step_fns:
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for fn in step_fns:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        return graphs
    except RuntimeError as exc:           # capture not possible here
        log(f"graph capture failed, timing eager launches: {exc}")
        return None


def time_graph_steps(graphs, steps):
    """Milliseconds per step over exactly `steps` replays (graph j % n for
    step j), bracketed by device synchronisation."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(steps):
        graphs[j % len(graphs)].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def percentiles(ms):
    """p10 / median / p90 of per-step event times (ms)."""
    q = np.percentile(np.asarray(ms, dtype=np.float64), [10, 50, 90])
    return {"p10": round(float(q[0]), 4), "p50": round(float(q[1]), 4),
            "p90": round(float(q[2]), 4)}


def cpu_baseline(wl, inp, tokens):
    """The oracle as it stands, on the first `tokens` tokens of the batch."""
    import oracle
    T = tokens
    x = np.ascontiguousarray(inp["x"][:T])
    t0 = time.perf_counter()
    if wl.router == "gemm":
        l64 = oracle.router_logits(x, inp["w_router"], inp.get("bias"))
        l32 = l64.astype(np.float32)
    else:
        l32 = np.ascontiguousarray(inp["logits"][:T])
    idx, w = oracle.topk_softmax(l32, wl.k)
    oracle.moe_tokens(x, idx, w, np.arange(T), wl.e_begin, wl.n_local,
                      inp["w_gate"], inp["w_up"], inp["w_down"])
    dt = time.perf_counter() - t0
    local = (idx >= wl.e_begin) & (idx < wl.e_begin + wl.n_local)
    rows = int(local.sum())
    flop = 6.0 * rows * wl.H * wl.I
    if wl.router == "gemm":
        flop += 2.0 * T * wl.H * wl.E
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {T} tokens of the batch ({rows} token-expert rows): "
                      f"fp64 router logits + top-k + per-token SwiGLU FFN of the "
                      f"chosen local experts + weighted sum; {dt:.1f} s"}


def cpu_baseline_mx(wl, inp, x_perm, offsets, s_perm, dy, rows, inter):
    """The oracle's MXFP8 step on a slice: the first `rows` rows of expert 0
    and its first `inter` intermediate channels (weights sliced to match)."""
    import oracle
    r = min(rows, int(offsets[1]))
    sl = slice(0, inter)
    wg = np.ascontiguousarray(inp["w_gate"][:1, sl, :])
    wu = np.ascontiguousarray(inp["w_up"][:1, sl, :])
    wd = np.ascontiguousarray(inp["w_down"][:1, :, sl])
    t0 = time.perf_counter()
    oracle.mxfp8_mlp_step(x_perm[:r], np.array([0, r]), s_perm[:r], wg, wu, wd,
                          dy[:r])
    dt = time.perf_counter() - t0
    flop = 18.0 * r * wl.H * inter
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{r} rows of expert 0 with its first {inter} of {wl.I} "
                      f"intermediate channels: fp64 MX quantisation of every "
                      f"GEMM operand (weights included), forward, dgrad and "
                      f"wgrad; {dt:.1f} s"}


def run_mx(args, wl, dev):
    """MXFP8 grouped-MLP training step: permute, quantise x, forward (gate/up
    + SwiGLU x scale, then down), backward (down + SwiGLU backward, then
    gate/up data and weight gradients).  Routing runs before timing; the
    master weights are quantised once per step in training, timed apart."""
    log(f"workload {wl.name}: generating inputs")
    t0 = time.time()
    inp = synth.make_inputs(wl, with_weights=False)
    d = {k: to_dev(v, dev) for k, v in inp.items()}
    W = {k: torch.empty(shape, dtype=torch.bfloat16, device=dev) for k, shape in
         (("w_gate", (wl.n_local, wl.I, wl.H)), ("w_up", (wl.n_local, wl.I, wl.H)),
          ("w_down", (wl.n_local, wl.H, wl.I)))}
    host_w = {k: [] for k in W}
    for e0 in range(0, wl.n_local, 2):
        e1 = min(wl.n_local, e0 + 2)
        part = synth.make_weights(wl, range(wl.e_begin + e0, wl.e_begin + e1))
        for key in W:
            W[key][e0:e1].copy_(to_dev(part[key], dev))
            host_w[key].append(part[key])
    for key in host_w:
        inp[key] = np.concatenate(host_w[key])
    T, k, H, I, n = wl.T, wl.k, wl.H, wl.I, wl.n_local
    F = T * k
    logits = d["logits"].clone()
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    moe.route_topk(k, logits=logits, topk_idx=topk_idx, topk_w=topk_w)
    pout = moe.PermuteOut(T, k, H, n, torch.bfloat16, dev)
    moe.permute(topk_idx, d["x"], wl.e_begin, n, topk_w=topk_w, out=pout)
    torch.cuda.synchronize()
    R = int(pout.offsets[-1].item())
    dy_host = synth.make_dy(wl, R)
    dy = torch.zeros((F, H), dtype=torch.bfloat16, device=dev)
    dy[:R].copy_(to_dev(dy_host, dev))
    log(f"inputs ready in {time.time() - t0:.1f} s, R = {R}")

    # Buffers and workspaces, allocated once.
    bf = torch.bfloat16
    xq = torch.empty((F, H), dtype=torch.uint8, device=dev)
    xs = torch.empty((F, H // 32), dtype=torch.uint8, device=dev)
    a = torch.empty((F, I), dtype=bf, device=dev)
    gu = torch.empty((F, 2 * I), dtype=bf, device=dev)
    y = torch.empty((F, H), dtype=bf, device=dev)
    dx = torch.empty((F, H), dtype=bf, device=dev)
    ds = torch.empty(F, dtype=torch.float32, device=dev)
    dwg = torch.empty((n, I, H), dtype=bf, device=dev)
    dwu = torch.empty_like(dwg)
    dwd = torch.empty((n, H, I), dtype=bf, device=dev)
    L = moe.lib()
    ws_f = torch.empty(L.moe_grouped_mlp_mxfp8_fwd_workspace_bytes(F, n, H, I),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(L.moe_grouped_mlp_mxfp8_bwd_workspace_bytes(F, n, H, I),
                       dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    # per timed step: step start, gate/up start, gate/up end, step end
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
          for _ in range(args.steps)]
    qev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    mw_holder = {}

    def quant_masters():
        mw_holder["mw"] = moe.MxWeights(W["w_gate"], W["w_up"], W["w_down"])

    def step(timed_ev=None):
        mw = mw_holder["mw"]
        if timed_ev is not None:
            timed_ev[0].record(stream)
        moe.permute(topk_idx, d["x"], wl.e_begin, n, topk_w=topk_w, out=pout)
        moe.mxfp8_quantize(pout.x_perm, 0, codes=xq, scales=xs)
        if timed_ev is not None:
            timed_ev[1].record(stream)
        moe.mxfp8_mlp_fwd(xq, xs, pout.offsets, pout.s_perm, mw, a=a, gu=gu,
                          workspace=ws_f, down=False)
        if timed_ev is not None:
            timed_ev[2].record(stream)
        moe.mxfp8_mlp_fwd_down(pout.offsets, mw, ws_f, F, y=y)
        moe.mxfp8_mlp_bwd(dy, pout.x_perm, a, gu, pout.offsets, pout.s_perm,
                          mw, dx=dx, ds=ds, dw_gate=dwg, dw_up=dwu,
                          dw_down=dwd, workspace=ws_b)
        if timed_ev is not None:
            timed_ev[3].record(stream)

    quant_masters()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    qev[0].record(stream)
    quant_masters()
    qev[1].record(stream)
    torch.cuda.synchronize()
    master_ms = qev[0].elapsed_time(qev[1])

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    gu_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    step_pct = percentiles([e[0].elapsed_time(e[3]) for e in ev])
    graphs = None if args.no_graph else capture_steps([step])
    ms_step = time_graph_steps(graphs, args.steps) if graphs else ms_eager
    timing = TIMING_GRAPH if graphs else TIMING_EAGER
    if args.copy_probe_mb > 0:
        copy_probe(args.copy_probe_mb, dev)

    flop_fwd = 6.0 * R * H * I
    flop = 3.0 * flop_fwd                       # forward + dgrad + wgrad
    tflops = flop / (ms_step * 1e-3) / 1e12
    gu_flop = 4.0 * R * H * I
    gu_tflops = gu_flop / (gu_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 (e4m3 + e8m0 per 32), fp32 accumulate",
        "data": "synthetic (seeded generator; random-init weights)",
        "config": {
            "workload": f"{wl.name}: MXFP8 grouped-MLP training step, T={T} "
                        f"hidden={H} intermediate={I} E={wl.E} top-{k}; "
                        f"permute + quantise x + forward + dgrad + wgrad",
            "rows": R,
            "router": "routed before timing",
        },
        "rows_per_s": round(R / (ms_step * 1e-3), 1),
        "step_mfma_frac_fp8": round(tflops / FP8_PEAK_TFLOPS, 4),
        "step_mfma_frac_bf16": round(tflops / BF16_PEAK_TFLOPS, 4),
        "master_quant_ms": round(master_ms, 4),
        "timing": timing,
        "ms_per_step_eager": round(ms_eager, 4),
        "step_ms_events": step_pct,
        "roofline": {
            "kernel": "MXFP8 grouped gate/up GEMM + SwiGLU x scale (forward)",
            "bound": "mfma",
            "achieved": round(gu_tflops, 2),
            "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gu_tflops / FP8_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(wl.name),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "avg_ms": round(gu_ms, 4),
        },
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle MXFP8 step on a slice")
        offs = pout.offsets.cpu().numpy()
        xp = pout.x_perm[:R].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        sp = pout.s_perm[:R].cpu().numpy().astype(np.float64)
        res["cpu_baseline"] = cpu_baseline_mx(wl, inp, xp, offs, sp, dy_host,
                                              rows=512, inter=2048)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4_full_bf16",
                    choices=["c4_full_bf16", "c2_ep64_bf16", "c3_ep8_bf16",
                             "c3_literal_ep8_bf16", "c5_shape_bf16",
                             "mid_bf16", "c5_mxfp8", "mid_mxfp8"])
    ap.add_argument("--cpu-tokens", type=int, default=1536)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gather", action="store_true",
                    help="full layer: permute writes x_perm and the gate/up "
                         "GEMM reads it, instead of reading token rows of x "
                         "through row_src (EP shares always read x_perm)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of replays of the step "
                         "captured in a HIP graph")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run one elementwise copy of this many "
                         "MiB (read + write) to calibrate HBM byte counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the expert layer; runs on "
              "more than one GPU are not part of this build (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if wl.dtype == "mxfp8":
        return run_mx(args, wl, dev)
    # Weight copies rotate across steps when the weights are small enough for
    # the 256 MB last-level cache to hold them between steps.
    wbytes = 3 * wl.n_local * wl.H * wl.I * 2
    copies = 1 if wbytes > 1.5e9 else 3
    log(f"workload {wl.name}: generating inputs ({wbytes / 1e9:.2f} GB of "
        f"weights x {copies})")
    t0 = time.time()
    inp, d, wcopies = make_device_workload(wl, dev, copies)
    log(f"inputs ready in {time.time() - t0:.1f} s")

    stream = torch.cuda.current_stream()
    T, k, H, I = wl.T, wl.k, wl.H, wl.I
    F = T * k
    # Buffers (capacity-sized), allocated once.
    logits = torch.empty((T, wl.E), dtype=torch.float32, device=dev)
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    # The full layer on one GPU reads token rows through row_src; an EP share
    # gets its rows already permuted by the dispatch, so it reads x_perm.
    gather = not args.no_gather and wl.n_local == wl.E
    pout = moe.PermuteOut(T, k, H, wl.n_local, torch.bfloat16, dev,
                          with_x=not gather)
    a = torch.empty((F, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((F, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = moe.ffn_workspace(F, wl.n_local, H, I, torch.bfloat16, dev)
    # per timed step: step start, gate/up start, gate/up end, down end, step end
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
          for _ in range(args.steps)]

    def route():
        if wl.router == "gemm":
            moe.route_topk(k, logits=logits, x=d["x"], w_router=d["w_router"],
                           bias=d.get("bias"), topk_idx=topk_idx, topk_w=topk_w)
        else:
            logits.copy_(d["logits"])
            moe.route_topk(k, logits=logits, topk_idx=topk_idx, topk_w=topk_w)

    def step(i, timed_ev=None):
        wg, wu, wd = wcopies[i % len(wcopies)]
        if timed_ev is not None:
            timed_ev[0].record(stream)
        if wl.router == "gemm":
            route()
        moe.permute(topk_idx, None if gather else d["x"], wl.e_begin,
                    wl.n_local, topk_w=topk_w, out=pout)
        if timed_ev is not None:
            timed_ev[1].record(stream)
        if gather:
            moe.grouped_gate_up_gather(d["x"], pout.row_src, k, pout.offsets,
                                       pout.s_perm, wg, wu, a=a, workspace=ws)
        else:
            moe.grouped_gate_up(pout.x_perm, pout.offsets, pout.s_perm, wg, wu,
                                a=a, workspace=ws)
        if timed_ev is not None:
            timed_ev[2].record(stream)
        moe.grouped_down(a, pout.offsets, wd, y=y, workspace=ws)
        if timed_ev is not None:
            timed_ev[3].record(stream)
        moe.unpermute_combine(y, pout.inv, out=out)
        if timed_ev is not None:
            timed_ev[4].record(stream)

    if wl.router != "gemm":
        route()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    R = int(pout.offsets[-1].item())
    n_touched = int((pout.counts > 0).sum().item())

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    gate_up_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    step_pct = percentiles([e[0].elapsed_time(e[4]) for e in ev])
    ffn_pct = percentiles([e[1].elapsed_time(e[3]) for e in ev])

    # the same steps replayed from captured graphs, one per weight copy
    graphs = (None if args.no_graph else
              capture_steps([lambda i=i: step(i) for i in range(len(wcopies))]))
    ms_step = time_graph_steps(graphs, args.steps) if graphs else ms_eager
    timing = TIMING_GRAPH if graphs else TIMING_EAGER

    if args.copy_probe_mb > 0:
        copy_probe(args.copy_probe_mb, dev)

    alg = algorithmic(wl, R, n_touched, gather)
    flop = alg["flop_ffn"] + alg["flop_router"]
    tflops = flop / (ms_step * 1e-3) / 1e12
    gu_gbs = alg["gate_up_bytes"] / (gate_up_ms * 1e-3) / 1e9
    gu_tflops = alg["gate_up_flop"] / (gate_up_ms * 1e-3) / 1e12
    # The gate/up kernel's bound: HBM below the bf16 ridge point (peak FLOP/s
    # over peak bytes/s), the matrix cores above it.
    ai = alg["gate_up_flop"] / alg["gate_up_bytes"]
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai < ridge:
        gate_up_bound = {"bound": "hbm", "achieved": round(gu_gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gu_gbs / HBM_PEAK_GBS, 4)}
    else:
        gate_up_bound = {"bound": "mfma", "achieved": round(gu_tflops, 2),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(gu_tflops / BF16_PEAK_TFLOPS, 4)}
    gate_up_bound["flop_per_byte"] = round(ai, 1)
    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator; random-init weights)",
        "config": {
            "workload": f"{wl.name}: T={T} hidden={H} intermediate={I} "
                        f"E={wl.E} top-{k}, local experts "
                        f"[{wl.e_begin},{wl.e_begin + wl.n_local})",
            "rows": R, "experts_touched": n_touched,
            "router": "router GEMM + softmax/top-k in the step"
                      if wl.router == "gemm" else "routed before timing",
            "gate_up_input": "token rows gathered on load through row_src"
                             if gather else "permuted copy x_perm",
        },
        "rows_per_s": round(R / (ms_step * 1e-3), 1),
        "step_hbm_gbs": round(alg["step_bytes"] / (ms_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(alg["step_bytes"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
        "timing": timing,
        "ms_per_step_eager": round(ms_eager, 4),
        "step_ms_events": step_pct,
        "ffn_ms_events": ffn_pct,
        "ffn_tflops_p50": round(alg["flop_ffn"] / (ffn_pct["p50"] * 1e-3) / 1e12, 2),
        "roofline": dict(**gate_up_bound, **{
            "kernel": "grouped gate/up GEMM + SwiGLU x scale",
            "traffic": measured_traffic(wl.name),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes": int(alg["gate_up_bytes"]),
            "avg_ms": round(gate_up_ms, 4),
            "gbs": round(gu_gbs, 1),
            "tflops": round(gu_tflops, 2),
            "mfma_frac": round(gu_tflops / BF16_PEAK_TFLOPS, 4),
        }),
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_tokens} tokens")
        res["cpu_baseline"] = cpu_baseline(wl, inp, min(args.cpu_tokens, T))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
