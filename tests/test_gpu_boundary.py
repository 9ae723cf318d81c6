"""Boundary behaviour on the device, through the C ABI.

- Top-k on logits holding NaN and infinities: indices bit-exact against the
  oracle's reading (NaN below -inf, ties to the lower index), weights close.
- moe_permute with expert indices outside [0, E): the slots are dropped like
  non-local ones (bit-exact against the oracle, which drops them the same
  way) and the workspace's error word reports MOE_DEVERR_EXPERT_INDEX; a
  clean call on the same workspace clears it.  Both dispatch paths: one
  workgroup (up to 8192 slots and 1024 local experts) and four launches.
- Grouped FFN with offsets past R_cap (or decreasing): segments are cut at
  R_cap, rows below it match the oracle, memory past the R_cap rows of a and
  y stays untouched, and the error word reports MOE_DEVERR_ROWS.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_router_amd as moe
import moe_synth as synth
import oracle as orc
from gpu_util import assert_close, print_case, to_dev, to_f64

pytestmark = pytest.mark.gpu


def test_topk_non_finite_logits():
    print_case("top-k, non-finite logits")
    rng = np.random.default_rng(21)
    T, E, k = 300, 40, 6
    l = rng.standard_normal((T, E)).astype(np.float32)
    specials = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0], dtype=np.float32)
    mask = rng.random((T, E)) < 0.3
    l[mask] = specials[rng.integers(len(specials), size=mask.sum())]
    l[0] = np.nan                                   # all NaN
    l[1] = -np.inf                                  # all -inf
    l[2, :] = np.nan; l[2, 7] = 1.0; l[2, 9] = -np.inf   # one finite logit
    l[3, :] = -np.inf; l[3, 5] = np.inf; l[3, 8] = np.inf
    l[4, :] = 0.0; l[4, ::2] = -0.0                 # signed zeros tie
    ridx, rw = orc.topk_softmax(l, k)
    idx, w, _ = moe.route_topk(k, logits=to_dev(l))
    moe.debug_sync()
    gi = idx.cpu().numpy()
    np.testing.assert_array_equal(gi, ridx)
    assert ((gi >= 0) & (gi < E)).all()
    assert all(len(set(r)) == k for r in gi.tolist())
    np.testing.assert_allclose(w.cpu().numpy(), rw, atol=2e-6)


def _perm_inputs(T, k, E, rng):
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    return idx


@pytest.mark.parametrize("T,k,E,e_begin,n_local", [
    (700, 4, 16, 4, 8),          # one workgroup (F <= 8192 slots)
    (2048, 4, 16, 4, 8),         # F = 8192, the one-workgroup limit
    (2049, 4, 16, 4, 8),         # F > 8192: four launches
    (40, 4, 2048, 100, 1100),    # more than 1024 local experts: four launches
])
def test_permute_out_of_range_index_sets_error_word(T, k, E, e_begin, n_local):
    print_case(f"permute, indices outside [0, E), T={T} k={k} E={E} n_local={n_local}")
    rng = np.random.default_rng(22)
    H = 64
    idx = _perm_inputs(T, k, E, rng)
    bad = idx.copy()
    pos = rng.choice(T * k, 37, replace=False)
    bad.reshape(-1)[pos] = rng.choice([-1, -7, E, E + 3, 1 << 30], 37)
    x = synth.normal_bf16(3, 1, 0, T * H, 0.0, 1.0).reshape(T, H)
    w = rng.random((T, k)).astype(np.float32)
    p = moe.permute(to_dev(bad), to_dev(x), e_begin, n_local,
                    topk_w=to_dev(w), E=E)
    code = moe.read_device_error(p.workspace)
    ref = orc.permute(bad, e_begin, n_local)
    assert code == moe.DEVERR_EXPERT_INDEX
    R = ref["R"]
    np.testing.assert_array_equal(p.counts.cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(p.offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(p.row_src.cpu().numpy()[:R], ref["row_src"])
    np.testing.assert_array_equal(p.inv.cpu().numpy(), ref["inv"])
    assert (p.inv.cpu().numpy().reshape(-1)[pos] == -1).all()
    # a clean call on the same workspace clears the word
    p2 = moe.permute(to_dev(idx), to_dev(x), e_begin, n_local,
                     topk_w=to_dev(w), E=E, out=p)
    assert moe.read_device_error(p2.workspace) == 0
    ref2 = orc.permute(idx, e_begin, n_local)
    np.testing.assert_array_equal(p2.inv.cpu().numpy(), ref2["inv"])


def test_permute_empty_batch_clears_error_word():
    print_case("permute, T = 0 after an error")
    dev = "cuda"
    bad = torch.full((3, 2), 99, dtype=torch.int32, device=dev)
    p = moe.permute(bad, None, 0, 4, E=8)
    assert moe.read_device_error(p.workspace) == moe.DEVERR_EXPERT_INDEX
    empty = torch.empty((0, 2), dtype=torch.int32, device=dev)
    q = moe.PermuteOut(0, 2, 64, 4, torch.bfloat16, dev, with_x=False)
    q.workspace = p.workspace
    moe.permute(empty, None, 0, 4, E=8, out=q)
    assert moe.read_device_error(p.workspace) == 0


def _ffn_case(dtype, H, I, n_local, rng):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def draw(shape, std, seed, stream):
        n = int(np.prod(shape))
        if dtype == "bf16":
            return synth.normal_bf16(seed, stream, 0, n, 0.0, std).reshape(shape)
        return synth.normal_f32(seed, stream, 0, n, 0.0, std).reshape(shape)

    wg = draw((n_local, I, H), 0.05, 5, 10)
    wu = draw((n_local, I, H), 0.05, 5, 11)
    wd = draw((n_local, H, I), 0.05, 5, 12)
    return tdt, wg, wu, wd, draw


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("offsets,R_cap", [
    ([0, 40, 100, 170], 130),          # last segment runs past R_cap
    ([0, 300, 300, 300], 200),         # first segment already does
    ([0, 50, 30, 90], 90),             # a decreasing pair: expert 1 empty
])
def test_grouped_ffn_rows_past_capacity(dtype, offsets, R_cap):
    print_case("ffn past R_cap", dtype, offsets, R_cap)
    rng = np.random.default_rng(23)
    H, I, n_local, guard = 128, 192, 3, 16
    tdt, wg, wu, wd, draw = _ffn_case(dtype, H, I, n_local, rng)
    xp = draw((R_cap, H), 1.0, 6, 1)
    s = rng.random(R_cap).astype(np.float32)
    dev = "cuda"
    sentinel = 1024.0                 # exact in bf16
    a_full = torch.full((R_cap + guard, I), sentinel, dtype=tdt, device=dev)
    y_full = torch.full((R_cap + guard, H), sentinel, dtype=tdt, device=dev)
    off = np.array(offsets, dtype=np.int32)
    ws = moe.ffn_workspace(R_cap, n_local, H, I, tdt, dev)
    a, y = moe.grouped_ffn(to_dev(xp), to_dev(off), to_dev(s), to_dev(wg),
                           to_dev(wu), to_dev(wd), a=a_full[:R_cap],
                           y=y_full[:R_cap], workspace=ws)
    assert moe.read_device_error(ws) == moe.DEVERR_ROWS
    assert (a_full[R_cap:].float() == sentinel).all()
    assert (y_full[R_cap:].float() == sentinel).all()
    # rows below R_cap: expert e computes [b_e, e_e) with b_e = clamp(off[e])
    # and e_e = clamp(off[e+1]) but at least b_e; a row two segments claim
    # (decreasing offsets) holds an unspecified value, so only rows with one
    # owner are compared
    ex = np.full(R_cap, -1)
    owners = np.zeros(R_cap, dtype=int)
    for e in range(n_local):
        b = min(max(off[e], 0), R_cap)
        en = min(max(off[e + 1], b), R_cap)
        ex[b:en] = e
        owners[b:en] += 1
    rows = np.nonzero(owners == 1)[0]
    a_ref, y_ref = orc.expert_ffn_rows(xp[rows], ex[rows].astype(np.int32),
                                       s[rows].astype(np.float64), wg, wu, wd)
    assert_close(to_f64(a[rows]), a_ref, dtype, "a")
    assert_close(to_f64(y[rows]), y_ref, dtype, "y")
    # rows in no segment are never written
    idle = np.nonzero(owners == 0)[0]
    assert (a_full[idle].float() == sentinel).all()
    # a clean call clears the word
    good = np.minimum(off, R_cap)
    good = np.maximum.accumulate(good).astype(np.int32)
    moe.grouped_ffn(to_dev(xp), to_dev(good), to_dev(s), to_dev(wg),
                    to_dev(wu), to_dev(wd), a=a_full[:R_cap], y=y_full[:R_cap],
                    workspace=ws)
    assert moe.read_device_error(ws) == 0
