"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
FLOP and byte counts the roofline divides by, the percentile summary and the
source-hash guard on the stored counter bytes."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import moe_synth as synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_counts_full_layer():
    wl = synth.WORKLOADS["c4_full_bf16"]
    R, H, I, T = 65536, wl.H, wl.I, wl.T
    a = bench.algorithmic(wl, R, 256, gather=True)
    assert a["flop_ffn"] == 6.0 * R * H * I
    assert a["flop_router"] == 2.0 * T * H * wl.E
    assert a["gate_up_flop"] == 4.0 * R * H * I
    # every touched expert's gate and up weights once, x rows once, a once
    assert a["gate_up_bytes"] == 2 * 256 * H * I * 2 + R * H * 2 + R * I * 2
    # all three weight sets, x rows read once (gathered), a and y written and
    # read, out written, plus the router's x, W_r and logits traffic
    step = (3 * 256 * H * I * 2 + R * H * 2 + 2 * R * I * 2 + 2 * R * H * 2
            + T * H * 2 + T * H * 2 + wl.E * H * 2 + 2 * T * wl.E * 4)
    assert a["step_bytes"] == step
    # an EP share reads x once in the permute and x_perm twice more
    b = bench.algorithmic(synth.WORKLOADS["c2_ep64_bf16"], 600, 4, gather=False)
    w2 = synth.WORKLOADS["c2_ep64_bf16"]
    assert b["step_bytes"] - b["gate_up_bytes"] > w2.T * w2.H * 2


def test_percentiles():
    p = bench.percentiles(list(range(1, 101)))
    assert p["p50"] == 50.5 and p["p10"] < p["p50"] < p["p90"]
    assert bench.percentiles([2.0] * 7) == {"p10": 2.0, "p50": 2.0, "p90": 2.0}


def test_stored_profile_follows_the_kernel_sources():
    # the stored figures are reported while the dominant kernel's sources
    # hash to the recorded value, and not for workloads without a record
    rec = bench.measured_profile("c4_full_bf16")
    assert rec is None or (rec["bytes"] > 0 and rec["avg_ms"] > 0)
    assert bench.measured_profile("no_such_workload") is None


def test_profile_fields():
    rec = {"avg_ms": 2.0, "mfma_busy": 0.5, "clock_ghz": 1.4, "wait_frac": 0.2,
           "profile": "profiles/x.md"}
    f = bench.profile_fields(rec, 8e9, 8000.0, 1e9)  # 8 GB in 2 ms
    assert f["achieved"] == 4000.0 and f["frac"] == 0.5
    assert f["summary"] == "profiles/x.md"
    assert bench.profile_fields(None, 1.0, 1.0, 1.0) is None
