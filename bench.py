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
TIMING_GRAPH = ("K steps replayed from HIP graphs that each hold up to 8 consecutive "
                "steps (same kernels, no host launch between them), after W eager "
                "warmup steps and K eager steps timed with HIP events")
TIMING_EAGER = "K eager steps"


def measured_profile(workload):
    """The dominant kernel's figures from the committed rocprofv3 runs
    (profiles/kernel_profile.json: timed-dispatch average duration, HBM
    bytes from FETCH_SIZE / WRITE_SIZE, MFMA ops, clock and busy fraction,
    wait fraction), or None when there are none or the kernel's sources
    changed since they were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "kernel_profile.json")
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
    return rec


def profile_fields(rec, amount, peak, unit_scale):
    """The roofline's profile-derived figures: `amount` (algorithmic bytes or
    FLOPs per launch) over the profiled average duration against `peak` (in
    units of unit_scale per second), beside the counters."""
    if rec is None:
        return None
    achieved = amount / (rec["avg_ms"] * 1e-3) / unit_scale
    return {"avg_ms": rec["avg_ms"], "achieved": round(achieved, 1),
            "frac": round(achieved / peak, 4),
            "mfma_busy": rec["mfma_busy"], "clock_ghz": rec["clock_ghz"],
            "wait_frac": rec["wait_frac"], "summary": rec["profile"]}


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
    # the fused FFN kernel: all weights, the rows of x, a written and read
    # back, y written
    fused_bytes = (w_bytes + R * H * act + 2 * R * I * act + R * H * act)
    return dict(flop_ffn=flop_ffn, flop_router=flop_router,
                gate_up_flop=4.0 * R * H * I, gate_up_bytes=gate_up_bytes,
                fused_bytes=fused_bytes, step_bytes=step_bytes)


# Consecutive steps captured in one HIP graph: a model replays many MoE
# layers inside one graph, so the step's kernels follow each other without a
# host launch between steps.
GRAPH_STEPS = 8


def capture_steps(step_fn, n_steps, period=1):
    """HIP graphs that hold consecutive steps: step_fn(j) runs step j (with
    preallocated buffers; j % period selects the rotated weight copy).
    Returns (graph of GRAPH_STEPS steps or fewer, steps in it, graph of the
    remaining n_steps % that many steps or None), or None when capture is
    not possible here."""
    per = max(1, min(GRAPH_STEPS, n_steps))
    per -= per % period if per >= period else 0
    per = max(per, 1)
    rest = n_steps % per
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for j in range(per):
                step_fn(j)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()

        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for j in range(n):
                    step_fn(j)
            return g

        full = capture(per)
        tail = capture(rest) if rest else None
        full.replay()
        if tail is not None:
            tail.replay()
        torch.cuda.synchronize()
        return full, per, tail
    except RuntimeError as exc:           # capture not possible here
        log(f"graph capture failed, timing eager launches: {exc}")
        return None


def time_graph_steps(graphs, steps):
    """Milliseconds per step over exactly `steps` steps replayed from the
    captured graphs, bracketed by device synchronisation."""
    full, per, tail = graphs
    n_full = steps // per
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_full):
        full.replay()
    if tail is not None:
        tail.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def percentiles(ms):
    """p10 / median / p90 of per-step event times (ms)."""
    q = np.percentile(np.asarray(ms, dtype=np.float64), [10, 50, 90])
    return {"p10": round(float(q[0]), 4), "p50": round(float(q[1]), 4),
            "p90": round(float(q[2]), 4)}


def host_cpu():
    """The host's CPU model and logical CPU count (the oracle's threads are
    reported as `cores`)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


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
            "kind": "oracle", **host_cpu(),
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
            "kind": "oracle", **host_cpu(),
            "sample": f"{r} rows of expert 0 with its first {inter} of {wl.I} "
                      f"intermediate channels: fp64 MX quantisation of every "
                      f"GEMM operand (weights included), forward, dgrad and "
                      f"wgrad; {dt:.1f} s"}


def run_mx(args, wl, dev, cpu=True):
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
    moe.permute(topk_idx, d["x"], wl.e_begin, n, topk_w=topk_w, out=pout, E=wl.E)
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
    gu = torch.empty((F, 2 * I), dtype=torch.float32, device=dev)
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
        moe.permute(topk_idx, d["x"], wl.e_begin, n, topk_w=topk_w, out=pout, E=wl.E)
        moe.mxfp8_quantize(pout.x_perm, 0, codes=xq, scales=xs)
        if timed_ev is not None:
            timed_ev[1].record(stream)
        moe.mxfp8_mlp_fwd(xq, xs, pout.offsets, pout.s_perm, mw, a=a, gu=gu,
                          workspace=ws_f, down=False)
        if timed_ev is not None:
            timed_ev[2].record(stream)
        moe.mxfp8_mlp_fwd_down(pout.offsets, mw, ws_f, F, y=y)
        moe.mxfp8_mlp_bwd(dy, pout.x_perm, gu, pout.offsets, pout.s_perm,
                          mw, dx=dx, ds=ds, dw_gate=dwg, dw_up=dwu,
                          dw_down=dwd, workspace=ws_b,
                          grad_format=args.grad_format)
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
    graphs = None if args.no_graph else capture_steps(lambda j: step(), args.steps)
    ms_step = time_graph_steps(graphs, args.steps) if graphs else ms_eager
    timing = TIMING_GRAPH if graphs else TIMING_EAGER
    if args.copy_probe_mb > 0:
        copy_probe(args.copy_probe_mb, dev)

    # the fused backward alone in both gradient formats (eager, same inputs)
    bwd_ms = {}
    for gfmt in ("e4m3", "e5m2"):
        def bwd(g=gfmt):
            moe.mxfp8_mlp_bwd(dy, pout.x_perm, gu, pout.offsets, pout.s_perm,
                              mw_holder["mw"], dx=dx, ds=ds, dw_gate=dwg,
                              dw_up=dwu, dw_down=dwd, workspace=ws_b,
                              grad_format=g)
        bwd()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            bwd()
        e1.record(stream)
        torch.cuda.synchronize()
        bwd_ms[gfmt] = round(e0.elapsed_time(e1) / args.steps, 4)

    flop_fwd = 6.0 * R * H * I
    flop = 3.0 * flop_fwd                       # forward + dgrad + wgrad
    tflops = flop / (ms_step * 1e-3) / 1e12
    gu_flop = 4.0 * R * H * I
    gu_tflops = gu_flop / (gu_ms * 1e-3) / 1e12
    prof = measured_profile(wl.name)
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
        "dtype": ("mxfp8 (e4m3 + e8m0 per 32), fp32 accumulate" if args.grad_format == "e4m3"
                  else "mxfp8 (e4m3; e5m2 gradients; e8m0 per 32), fp32 accumulate"),
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
        "backward_ms_by_grad_format": bwd_ms,
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
            "traffic": (prof or {}).get("bytes"),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "avg_ms": round(gu_ms, 4),
            "profile": profile_fields(prof, gu_flop, FP8_PEAK_TFLOPS, 1e12),
        },
    }
    if cpu:
        log("cpu baseline: oracle MXFP8 step on a slice")
        offs = pout.offsets.cpu().numpy()
        xp = pout.x_perm[:R].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        sp = pout.s_perm[:R].cpu().numpy().astype(np.float64)
        res["cpu_baseline"] = cpu_baseline_mx(wl, inp, xp, offs, sp, dy_host,
                                              rows=512, inter=2048)
    return res


def dense_vs_library(args, dev):
    """Calibration, not the step: one dense bf16 GEMM, C[M, N] = A[M, K] .
    W[N, K]^T with M 32768, N 16384, K 4096, by this library's grouped GEMM
    (one expert, the down projection's call) and by torch.mm (the vendor
    BLAS), each timed with HIP events over K calls after W warm-up
    calls.  The rocprofv3 counters of both kernels come from profiling this
    mode."""
    M, N, K = 32768, 16384, 4096
    g = torch.Generator(device="cpu").manual_seed(0)
    a = (torch.randn(M, K, generator=g) * 0.5).to(torch.bfloat16).to(dev)
    w = (torch.randn(1, N, K, generator=g) * 0.02).to(torch.bfloat16).to(dev)
    offsets = torch.tensor([0, M], dtype=torch.int32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = moe.ffn_workspace(M, 1, N, K, torch.bfloat16, dev)
    lib_out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def ours():
        moe.grouped_down(a, offsets, w, y=y, workspace=ws)

    wt = w[0].t()  # a transposed view: the BLAS reads W K-contiguous as it is

    def library():
        torch.mm(a, wt, out=lib_out)

    res = {}
    for name, fn in (("grouped_gemm", ours), ("library_linear", library)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        res[name] = {"ms": round(ms, 4),
                     "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}
    err = (y.float() - lib_out.float()).abs().max().item()
    ref = lib_out.float().pow(2).mean().sqrt().item()
    return {"mode": "dense_vs_library", "M": M, "N": N, "K": K,
            "dtype": "bf16", **res,
            "max_abs_diff_over_rms": round(err / ref, 5),
            "what": "calibration of the bf16 GEMM mainloop against the vendor "
                    "library on one dense GEMM; not a step of the path"}


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
                    help="permute writes x_perm and the gate/up GEMM reads "
                         "it, instead of reading token rows of x through "
                         "row_src")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of replays of the step "
                         "captured in a HIP graph")
    ap.add_argument("--no-extra", action="store_true",
                    help="default workload only: skip the EP8 share, the EP64 "
                         "share and the MXFP8 step timed after it")
    ap.add_argument("--no-eplb", action="store_true",
                    help="skip the EP8 load-balancing comparison of the full layer")
    ap.add_argument("--grad-format", choices=("e4m3", "e5m2"), default="e4m3",
                    help="MXFP8 step: element format of the backward's "
                         "gradient operands (dY, dg, du)")
    ap.add_argument("--ffn", choices=("grouped", "fused"), default="grouped",
                    help="bf16 FFN path: the grouped GEMMs (default) or the "
                         "one-launch FFN on the same tiles (about 2%% slower on "
                         "the EP8 share, 9%% slower on the EP64 share)")
    ap.add_argument("--no-loop", action="store_true",
                    help="skip the per-expert-loop comparison of the grouped FFN")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run one elementwise copy of this many "
                         "MiB (read + write) to calibrate HBM byte counters")
    ap.add_argument("--dense-vs-library", action="store_true",
                    help="calibration instead of the benchmark: one dense bf16 "
                         "GEMM by this library and by the vendor BLAS")
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
    if args.dense_vs_library:
        print(json.dumps(dense_vs_library(args, dev)), flush=True)
        return
    cpu = not args.no_cpu_baseline
    if wl.dtype == "mxfp8":
        res = run_mx(args, wl, dev, cpu=cpu)
    else:
        res = run_bf16(args, wl, dev, cpu=cpu, loop=not args.no_loop)
    if args.workload == "c4_full_bf16" and not args.no_extra:
        # The other configurations of the metric, timed the same way (no CPU
        # baseline, which is taken on the main workload only).
        extra = {}
        for name in ("c3_ep8_bf16", "c2_ep64_bf16", "c5_mxfp8"):
            torch.cuda.empty_cache()
            w2 = synth.WORKLOADS[name]
            if w2.dtype == "mxfp8":
                r = run_mx(args, w2, dev, cpu=False)
            else:
                r = run_bf16(args, w2, dev, cpu=False, loop=not args.no_loop)
            extra[name] = compact(r)
        res["extra_workloads"] = extra
    print(json.dumps(res), flush=True)


def compact(r):
    """The figures of a result that the extra workloads report."""
    keep = ("value", "unit", "ms_per_step", "ms_per_step_eager", "dtype",
            "rows_per_s", "step_hbm_gbs", "step_hbm_frac", "step_mfma_frac",
            "step_mfma_frac_fp8", "step_mfma_frac_bf16", "ffn_ms_events",
            "ffn_hbm_frac_p50",
            "step_ms_events", "loop_vs_grouped", "fused_vs_grouped",
            "master_quant_ms", "backward_ms_by_grad_format")
    out = {k: r[k] for k in keep if k in r}
    out["workload"] = r["config"]["workload"]
    out["rows"] = r["config"]["rows"]
    out["roofline"] = {k: v for k, v in r["roofline"].items()
                       if k not in ("traffic_unit",)}
    return out


def loop_vs_grouped(wl, x, topk_idx, topk_w, wcopies, steps, dev):
    """The grouped FFN (one launch sequence for all experts) against the
    per-expert loop (a launch sequence per expert, counts read back to the
    host each step, as a loop must) on the same permuted rows: gate/up +
    down, eager launches, mean over `steps` steps."""
    T, k, H, I, n = wl.T, wl.k, wl.H, wl.I, wl.n_local
    p = moe.PermuteOut(T, k, H, n, torch.bfloat16, dev)
    moe.permute(topk_idx, x, wl.e_begin, n, topk_w=topk_w, out=p, E=wl.E)
    F = T * k
    a = torch.empty((F, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((F, H), dtype=torch.bfloat16, device=dev)
    ws = moe.ffn_workspace(F, n, H, I, torch.bfloat16, dev)
    counts_host = torch.empty(n, dtype=torch.int32, pin_memory=True)

    def grouped(i):
        wg, wu, wd = wcopies[i % len(wcopies)]
        moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, wg, wu, wd, a=a, y=y,
                        workspace=ws)

    def looped(i):
        wg, wu, wd = wcopies[i % len(wcopies)]
        counts_host.copy_(p.counts)          # the loop needs the sizes on the host
        torch.cuda.current_stream().synchronize()
        moe.grouped_ffn_loop(p.x_perm, p.offsets, counts_host.tolist(),
                             p.s_perm, wg, wu, wd, a=a, y=y, workspace=ws)

    out = {}
    for name, fn in (("grouped", grouped), ("loop", looped)):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        out[f"{name}_ms"] = round((time.perf_counter() - t0) * 1e3 / steps, 4)
    nz = int((p.counts > 0).sum().item())
    out["loop_over_grouped"] = round(out["loop_ms"] / out["grouped_ms"], 3)
    out["experts_with_rows"] = nz
    out["what"] = ("gate/up + down on the same permuted rows; the loop issues "
                   "each expert's launches separately and reads the counts "
                   "back to the host every step")
    del p, a, y, ws
    return out


def fused_vs_grouped(wl, x, topk_idx, topk_w, wcopies, steps, dev):
    """The grouped FFN (plan + gate/up launch, plan + down launch) against
    the fused one-launch FFN on the same permuted rows, eager launches, mean
    over `steps` steps."""
    T, k, H, I, n = wl.T, wl.k, wl.H, wl.I, wl.n_local
    p = moe.PermuteOut(T, k, H, n, torch.bfloat16, dev)
    moe.permute(topk_idx, x, wl.e_begin, n, topk_w=topk_w, out=p, E=wl.E)
    F = T * k
    a = torch.empty((F, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((F, H), dtype=torch.bfloat16, device=dev)
    ws = moe.ffn_workspace(F, n, H, I, torch.bfloat16, dev)

    def grouped(i):
        wg, wu, wd = wcopies[i % len(wcopies)]
        moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, wg, wu, wd, a=a, y=y,
                        workspace=ws)

    def fused(i):
        wg, wu, wd = wcopies[i % len(wcopies)]
        moe.grouped_ffn_fused(p.x_perm, p.offsets, p.s_perm, wg, wu, wd, a=a,
                              y=y, workspace=ws)

    out = {}
    for name, fn in (("grouped", grouped), ("fused", fused)):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        out[f"{name}_ms"] = round((time.perf_counter() - t0) * 1e3 / steps, 4)
    out["grouped_over_fused"] = round(out["grouped_ms"] / out["fused_ms"], 3)
    out["rows_per_expert"] = round(float(p.offsets[-1].item()) / n, 2)
    out["what"] = "gate/up + down on the same permuted rows, eager launches"
    del p, a, y, ws
    return out


def eplb_ep8(wl, x, topk_idx, topk_w, weights, steps, dev, n_ranks=8):
    """The full layer's routing split over n_ranks EP ranks, each rank's
    share timed alone on this GPU (gate/up + down of its rows; HIP events,
    mean over `steps`).  In EP the ranks run at once, so the busiest rank
    sets the layer's time.  Two placements of the same routing:
      "as_drawn": experts keep their numbers (the Zipf ranks are a seeded
        shuffle, so hot experts are spread over the ranks);
      "hot_first": experts renumbered by decreasing load, so that plain EP
        puts the hottest E/G experts on rank 0 (the concentration the EPLB
        section describes).
    For each: plain EP (rank g owns experts [g E/G, (g+1) E/G)), the EPLB
    placement without spare slots, and EPLB with E/8 spare slots; the plans
    are made from this batch's per-expert counts."""
    T, k, H, I, E = wl.T, wl.k, wl.H, wl.I, wl.E
    wg, wu, wd = weights
    F = T * k
    a = torch.empty((F, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((F, H), dtype=torch.bfloat16, device=dev)
    st = torch.cuda.current_stream()

    def timed(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(steps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def shares(idx, counts, S):
        """Per-rank rows and FFN times; S = None: plain EP."""
        rows, ms, perm_ms, plan_ms = [], [], [], None
        if S is not None:
            plan = moe.eplb_plan(counts, S, n_ranks)
            plan_ms = timed(lambda: moe.eplb_plan(counts, S, n_ranks))
        per = (E if S is None else S) // n_ranks
        ws = moe.ffn_workspace(F, per, H, I, torch.bfloat16, dev)
        for g in range(n_ranks):
            if S is None:
                p = moe.permute(idx, x, g * per, per, topk_w=topk_w, E=E)
                sl = slice(g * per, (g + 1) * per)
                fn = lambda: moe.grouped_ffn(p.x_perm, p.offsets, p.s_perm, wg[sl],
                                             wu[sl], wd[sl], a=a, y=y, workspace=ws)
            else:
                p = moe.permute_replicated(idx, x, plan, g * per, per,
                                           topk_w=topk_w, E=E)
                perm_ms.append(timed(lambda: moe.permute_replicated(
                    idx, x, plan, g * per, per, topk_w=topk_w, E=E, out=p)))
                se = plan["slot_expert"][g * per:(g + 1) * per].contiguous()
                fn = lambda: moe.grouped_ffn_slots(p.x_perm, p.offsets, p.s_perm, se,
                                                   wg, wu, wd, a=a, y=y, workspace=ws)
            torch.cuda.synchronize()
            rows.append(int(p.offsets[-1].item()))
            ms.append(timed(fn))
            del p
        r = {"slots": E if S is None else S,
             "rows_per_rank": rows,
             "rows_max_over_mean": round(max(rows) / (sum(rows) / n_ranks), 4),
             "ffn_ms_max_rank": round(max(ms), 4),
             "ffn_ms_mean_rank": round(sum(ms) / n_ranks, 4)}
        if S is not None:
            r["plan_ms"] = round(plan_ms, 4)
            r["permute_ms_max_rank"] = round(max(perm_ms), 4)
        return r

    counts = torch.bincount(topk_idx.reshape(-1).long(), minlength=E).to(torch.int32)
    order = torch.argsort(counts, descending=True, stable=True)
    relabel = torch.empty_like(order)
    relabel[order] = torch.arange(E, device=dev)
    out = {"ranks": n_ranks, "experts": E}
    for name, idx in (("as_drawn", topk_idx),
                      ("hot_first", relabel[topk_idx.long()].to(torch.int32).contiguous())):
        c = torch.bincount(idx.reshape(-1).long(), minlength=E).to(torch.int32)
        res = {"plain_ep": shares(idx, c, None),
               "eplb_placement": shares(idx, c, E),
               "eplb_spare": shares(idx, c, E + E // 8)}
        base = res["plain_ep"]["ffn_ms_max_rank"]
        for key in ("eplb_placement", "eplb_spare"):
            res[key]["max_rank_speedup_over_plain"] = round(base / res[key]["ffn_ms_max_rank"], 3)
        out[name] = res
    out["what"] = ("each rank's share of this batch timed alone on this GPU; plans made "
                   "from this batch's counts (the loads they balance)")
    return out


def run_bf16(args, wl, dev, cpu=True, loop=True):
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
    # The gate/up GEMM reads the token rows through row_src (the permute
    # writes no x_perm), on the full layer and on the EP shares alike.
    gather = not args.no_gather
    fused = args.ffn == "fused"
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
                    wl.n_local, topk_w=topk_w, out=pout, E=wl.E)
        if timed_ev is not None:
            timed_ev[1].record(stream)
        if fused:
            if gather:
                moe.grouped_ffn_fused(d["x"], pout.offsets, pout.s_perm, wg, wu,
                                      wd, row_src=pout.row_src, k=k, a=a, y=y,
                                      workspace=ws)
            else:
                moe.grouped_ffn_fused(pout.x_perm, pout.offsets, pout.s_perm,
                                      wg, wu, wd, a=a, y=y, workspace=ws)
            if timed_ev is not None:
                timed_ev[2].record(stream)
                timed_ev[3].record(stream)
        elif timed_ev is None:
            # warm-up and captured steps: one call, one plan kernel for both
            # GEMMs
            if gather:
                moe.grouped_ffn_gather(d["x"], pout.row_src, k, pout.offsets,
                                       pout.s_perm, wg, wu, wd, a=a, y=y,
                                       workspace=ws)
            else:
                moe.grouped_ffn(pout.x_perm, pout.offsets, pout.s_perm, wg, wu,
                                wd, a=a, y=y, workspace=ws)
        else:
            # event-timed eager steps: gate/up and down as separate calls
            # (each with its plan kernel) so that an event sits between them
            if gather:
                moe.grouped_gate_up_gather(d["x"], pout.row_src, k, pout.offsets,
                                           pout.s_perm, wg, wu, a=a, workspace=ws)
            else:
                moe.grouped_gate_up(pout.x_perm, pout.offsets, pout.s_perm, wg,
                                    wu, a=a, workspace=ws)
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
              capture_steps(step, args.steps, len(wcopies)))
    ms_step = time_graph_steps(graphs, args.steps) if graphs else ms_eager
    timing = TIMING_GRAPH if graphs else TIMING_EAGER

    if args.copy_probe_mb > 0:
        copy_probe(args.copy_probe_mb, dev)

    res_eplb = None
    if wl.n_local == wl.E and not args.no_eplb:
        log(f"{wl.name}: EP8 shares, plain and balanced")
        res_eplb = eplb_ep8(wl, d["x"], topk_idx, topk_w, wcopies[0],
                            args.steps, dev)
    if loop:
        log(f"{wl.name}: per-expert loop against the grouped FFN")
        res_loop = loop_vs_grouped(wl, d["x"], topk_idx, topk_w, wcopies,
                                   args.steps, dev)
    res_fused = None
    if wl.n_local < wl.E:
        log(f"{wl.name}: fused one-launch FFN against the grouped FFN")
        res_fused = fused_vs_grouped(wl, d["x"], topk_idx, topk_w, wcopies,
                                     args.steps, dev)
    alg = algorithmic(wl, R, n_touched, gather)
    prof = measured_profile(wl.name)
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
    if fused:
        # one kernel streams every weight once: HBM-bound at these row counts
        f_gbs = alg["fused_bytes"] / (gate_up_ms * 1e-3) / 1e9
        gate_up_bound = {"bound": "hbm", "achieved": round(f_gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(f_gbs / HBM_PEAK_GBS, 4),
                         "flop_per_byte": round(alg["flop_ffn"] / alg["fused_bytes"], 1)}
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
            "ffn": "fused gate/up + down, one persistent launch" if fused
                   else "grouped gate/up GEMM, then grouped down GEMM",
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
        # the FFN's own bytes (every touched expert's weights once, the rows
        # of x read, a written and read back, y written) over its p50 time
        "ffn_hbm_frac_p50": round(alg["fused_bytes"] / (ffn_pct["p50"] * 1e-3) / 1e9
                                  / HBM_PEAK_GBS, 4),
        "roofline": dict(**gate_up_bound, **{
            "kernel": ("fused FFN (gate/up + SwiGLU x scale + down) with its plan kernel"
                       if fused else "grouped gate/up GEMM + SwiGLU x scale"),
            "traffic": None if fused else (prof or {}).get("bytes"),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "profile": None if fused else (
                profile_fields(prof, alg["gate_up_bytes"], HBM_PEAK_GBS, 1e9)
                if gate_up_bound["bound"] == "hbm" else
                profile_fields(prof, alg["gate_up_flop"], BF16_PEAK_TFLOPS, 1e12)),
            "algorithmic_bytes": int(alg["fused_bytes"] if fused else alg["gate_up_bytes"]),
            "avg_ms": round(gate_up_ms, 4),
            "gbs": round(gu_gbs, 1),
            "tflops": round(gu_tflops, 2),
            "mfma_frac": round(gu_tflops / BF16_PEAK_TFLOPS, 4),
        }),
    }
    if loop:
        res["loop_vs_grouped"] = res_loop
    if res_fused is not None:
        res["fused_vs_grouped"] = res_fused
    if res_eplb is not None:
        res["eplb_ep8"] = res_eplb
    if cpu:
        log(f"cpu baseline: oracle on {args.cpu_tokens} tokens")
        res["cpu_baseline"] = cpu_baseline(wl, inp, min(args.cpu_tokens, T))
    return res


if __name__ == "__main__":
    main()
