"""Pins of the oracle's expert-parallel load balancing (EPLB) against
brute force and invariants: the replica counts minimise the largest load
per copy; the row ranges of an expert's copies partition its rows; every
rank gets S/G slots; copies of one expert sit on distinct ranks when that
is possible; the dispatch equals a stable sort of the flat entries by the
slot that a direct reading of the plan assigns."""
import itertools

import numpy as np
import pytest

import oracle as orc


def _compositions(total, parts):
    """All ways to give `total` extra copies to `parts` experts."""
    for c in itertools.combinations(range(total + parts - 1), parts - 1):
        prev, out = -1, []
        for x in c + (total + parts - 1,):
            out.append(x - prev - 1)
            prev = x
        yield out


@pytest.mark.parametrize("seed", range(6))
def test_replication_minimises_the_largest_load_per_copy(seed):
    rng = np.random.default_rng(seed)
    E = 5
    extra = int(rng.integers(1, 6))
    counts = rng.integers(0, 60, E).astype(np.int32)
    p = orc.eplb_plan(counts, E + extra, 1)
    rep = p["rep"]
    assert rep.sum() == E + extra and (rep >= 1).all()
    got = max(c / r for c, r in zip(counts, rep))
    best = min(max(c / (1 + x) for c, x in zip(counts, xs))
               for xs in _compositions(extra, E))
    assert got == best
    # ties go to the lower expert index: an all-equal load replicates 0, 1, ...
    q = orc.eplb_plan(np.full(4, 10, np.int32), 6, 1)
    np.testing.assert_array_equal(q["rep"], [2, 2, 1, 1])


def _ranges(plan, counts):
    """Row range of every slot under `counts` (copy i of r of an expert with
    n rows: [floor(i n / r), floor((i+1) n / r)))."""
    lo = np.empty(len(plan["slot_expert"]), np.int64)
    hi = np.empty_like(lo)
    for s_, (e, i) in enumerate(zip(plan["slot_expert"], plan["slot_copy"])):
        lo[s_], hi[s_] = orc.copy_rows(int(counts[e]), int(plan["rep"][e]), int(i))
    return lo, hi


def test_copies_partition_each_experts_rows():
    counts = np.array([100, 7, 0, 33, 1, 64, 64, 2], np.int32)
    p = orc.eplb_plan(counts, 16, 4)
    lo, hi = _ranges(p, counts)
    for e in range(8):
        slots = p["rep_slot"][p["rep_first"][e]:p["rep_first"][e + 1]]
        assert (p["slot_expert"][slots] == e).all()
        np.testing.assert_array_equal(p["slot_copy"][slots], np.arange(len(slots)))
        assert lo[slots][0] == 0 and hi[slots][-1] == counts[e]
        np.testing.assert_array_equal(lo[slots][1:], hi[slots][:-1])
        sizes = hi[slots] - lo[slots]
        assert sizes.max() - sizes.min() <= 1           # as even as possible


def test_placement_fills_ranks_and_spreads_copies():
    rng = np.random.default_rng(9)
    E, S, G = 32, 40, 8
    counts = (1000 * (1 + np.arange(E)) ** -1.2).astype(np.int32)
    rng.shuffle(counts)
    p = orc.eplb_plan(counts, S, G)
    per = S // G
    rank = np.arange(S) // per
    # every rank holds exactly S/G slots and every slot exactly one copy
    assert sorted(p["rep_slot"].tolist()) == list(range(S))
    for e in range(E):
        r = rank[p["rep_slot"][p["rep_first"][e]:p["rep_first"][e + 1]]]
        assert len(set(r.tolist())) == len(r)           # distinct ranks
    # inside a rank, slots run in increasing (expert, copy) order
    key = p["slot_expert"] * 1000 + p["slot_copy"]
    for g in range(G):
        assert (np.diff(key[g * per:(g + 1) * per]) > 0).all()
    # the greedy bound: no rank exceeds the mean by more than the largest copy
    lo, hi = _ranges(p, counts)
    loads = np.array([(hi - lo)[g * per:(g + 1) * per].sum() for g in range(G)])
    assert loads.max() <= loads.mean() + (hi - lo).max()
    # and balancing helps: the plain split (32/8 = 4 experts a rank) is worse
    assert loads.max() < counts.reshape(G, -1).sum(1).max()


def test_placement_hand_example():
    # 4 experts with rows 9, 5, 4, 2; 6 slots on 3 ranks of 2.
    # Replication: 9/1 is the largest load per copy -> expert 0 gets a second
    # copy (4.5 each); then 5/1 -> expert 1 (2.5 each).  Copies and sizes:
    # e0 [0,4) 4, e0 [4,9) 5, e1 [0,2) 2, e1 [2,5) 3, e2 4, e3 2; placed in
    # the order e0[4,9) 5, e0[0,4) 4, e2 4, e1[2,5) 3, e1[0,2) 2, e3 2:
    #   e0[4,9) -> rank 0 (all empty, lowest rank)           loads 5 0 0
    #   e0[0,4) -> rank 1 (rank 0 holds e0)                  loads 5 4 0
    #   e2      -> rank 2                                    loads 5 4 4
    #   e1[2,5) -> rank 1 (4 ties 4: lower rank)             loads 5 7 4, rank 1 full
    #   e1[0,2) -> rank 2 (rank 1 full; 4 < 5)               loads 5 7 6, rank 2 full
    #   e3      -> rank 0 (the only free slot)
    p = orc.eplb_plan(np.array([9, 5, 4, 2], np.int32), 6, 3)
    np.testing.assert_array_equal(p["rep"], [2, 2, 1, 1])
    rank = np.arange(6) // 2
    where = {(int(p["slot_expert"][s]), int(p["slot_copy"][s])): int(rank[s]) for s in range(6)}
    assert where == {(0, 1): 0, (0, 0): 1, (2, 0): 2, (1, 1): 1, (1, 0): 2, (3, 0): 0}


@pytest.mark.parametrize("G,S", [(1, 8), (4, 12), (4, 16)])
def test_replicated_permute_is_a_stable_sort_by_slot(G, S):
    rng = np.random.default_rng(S + G)
    T, k, E = 60, 3, 8
    idx = np.stack([rng.choice(E, k, replace=False, p=np.arange(1, E + 1) / 36.0)
                    for _ in range(T)]).astype(np.int32)
    idx[5, 1] = E + 2                                   # outside [0, E): dropped
    # the plan comes from other (earlier) loads than the routing dispatched
    p = orc.eplb_plan(rng.integers(0, 50, E).astype(np.int32), S, G)
    per = S // G
    counts = np.bincount(idx[(idx >= 0) & (idx < E)], minlength=E)
    lo, hi = _ranges(p, counts)
    # slot of every flat entry by a direct reading of the plan
    flat = idx.reshape(-1)
    seen = np.zeros(E, int)
    slot = np.full(T * k, -1)
    for f, e in enumerate(flat):
        if not 0 <= e < E:
            continue
        q = seen[e]; seen[e] += 1
        for c in range(p["rep_first"][e], p["rep_first"][e + 1]):
            s_ = p["rep_slot"][c]
            if lo[s_] <= q < hi[s_]:
                slot[f] = s_
    covered = np.zeros(T * k, int)
    for g in range(G):
        r = orc.permute_replicated(idx, E, p, g * per, per)
        local = np.nonzero((slot >= g * per) & (slot < (g + 1) * per))[0]
        want = local[np.argsort(slot[local], kind="stable")]
        np.testing.assert_array_equal(r["row_src"], want)
        np.testing.assert_array_equal(r["counts"], (hi - lo)[g * per:(g + 1) * per])
        inv = r["inv"].reshape(-1)
        assert (inv[want] == np.arange(len(want))).all()
        covered[want] += 1
    assert (covered == (slot >= 0)).all()               # each entry on one rank
    assert covered[5 * k + 1] == 0
