"""Every unit of a large grouped launch is run exactly once.

Launches with at least 8 units per workgroup hand their units out through
per-XCD claim counters (with claims across XCDs at the end) instead of the
static walk; the parity tests at full size sample rows.  Here the inputs are
one-hot rows, so every output element has a cheap exact reference and all
of them are checked:
- gate/up with x row r equal to the unit vector at h_r: g and u are the
  weight columns W_gate[e, :, h_r] and W_up[e, :, h_r] exactly (one bf16
  product per sum), and a = s * SiLU(g) * u is compared with the oracle's
  ScaledSwiGLU of those columns, every row;
- down with a row r equal to the unit vector at i_r: y row r is the weight
  column W_down[e, :, i_r], bit for bit.
8 experts of 2048 rows, H = 4096, I = 2048: 2048 units in each launch, 8
per workgroup on 256 compute units.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_router_amd as moe
import oracle as orc
from gpu_util import assert_close, print_case, to_f64

pytestmark = pytest.mark.gpu

G, ROWS, H, I = 8, 2048, 4096, 2048


def _weights(seed, shape):
    gen = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=gen) * 0.5).to(torch.bfloat16)


def test_claimed_units_cover_every_tile():
    print_case(f"one-hot grouped gate/up and down, {G} x {ROWS} rows, H={H} I={I}")
    dev = "cuda"
    R = G * ROWS
    r = np.arange(R)
    e = r // ROWS
    h = (r * 7 + e) % H
    i = (r * 5 + 3) % I
    wg = _weights(1, (G, I, H))
    wu = _weights(2, (G, I, H))
    wd = _weights(3, (G, H, I))
    s = (np.random.default_rng(4).random(R) + 0.5).astype(np.float32)
    x = torch.zeros((R, H), dtype=torch.bfloat16)
    x[torch.from_numpy(r), torch.from_numpy(h)] = 1.0
    a_in = torch.zeros((R, I), dtype=torch.bfloat16)
    a_in[torch.from_numpy(r), torch.from_numpy(i)] = 1.0
    offsets = torch.arange(0, R + 1, ROWS, dtype=torch.int32)

    ws = moe.ffn_workspace(R, G, H, I, torch.bfloat16, dev)
    a = moe.grouped_gate_up(x.to(dev), offsets.to(dev),
                            torch.from_numpy(s).to(dev), wg.to(dev),
                            wu.to(dev), workspace=ws)
    y = moe.grouped_down(a_in.to(dev), offsets.to(dev), wd.to(dev),
                         workspace=ws)
    moe.debug_sync()

    # references from the inputs alone
    te, th, ti = (torch.from_numpy(v) for v in (e, h, i))
    g_ref = wg[te, :, th].double().numpy()
    u_ref = wu[te, :, th].double().numpy()
    a_ref = orc.swiglu(g_ref, u_ref, s.astype(np.float64))
    err = assert_close(to_f64(a), a_ref, "bf16", "a (one-hot gate/up)")
    print(f"a: max|err|/RMS = {err:.3e}")
    y_ref = wd[te, :, ti]
    assert torch.equal(y.cpu().view(torch.int16), y_ref.view(torch.int16)), \
        "y (one-hot down) differs from the weight columns"
