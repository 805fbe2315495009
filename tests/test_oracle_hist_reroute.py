"""Pins for the oracle's histogram (A1) and reroute (A3).

Histogram: the count of each expert ID is fixed by its definition, so it is
checked against numpy's bincount and the count of valid pairs.  Reroute: every
pair must go to an instance of its own logical expert (the balancing keeps the
model mathematically unchanged -- UltraEP article, design principles), each
instance must receive exactly its quota (per-instance quota -- UltraEP article,
key designs), and the assignment must follow flat (rank, token, k) order.  An
independent construction through a stable argsort reproduces the whole output.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W


def _rand_ids(rng, n, E, pad=0.05, bad=0.02):
    ids = rng.integers(0, E, size=n).astype(np.int32)
    m = rng.random(n)
    ids[m < pad] = -1 - rng.integers(0, 3, size=int((m < pad).sum()))
    sel = (m >= pad) & (m < pad + bad)
    ids[sel] = E + rng.integers(0, 4, size=int(sel.sum()))
    return ids


@pytest.mark.parametrize("seed", range(5))
def test_histogram_matches_bincount(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 400))
    n = int(rng.integers(0, 50000))
    ids = _rand_ids(rng, n, E)
    load, bad = oracle.histogram(ids, E)
    valid = ids[(ids >= 0) & (ids < E)]
    np.testing.assert_array_equal(load, np.bincount(valid, minlength=E))
    assert load.sum() == valid.size
    assert bad == int((ids >= E).sum())


def test_histogram_empty_and_all_padding():
    load, bad = oracle.histogram(np.zeros(0, np.int32), 7)
    assert load.tolist() == [0] * 7 and bad == 0
    load, bad = oracle.histogram(np.full(100, -1, np.int32), 7)
    assert load.sum() == 0 and bad == 0


def test_histogram_on_workload_ids():
    wl = W.get("qwen3_235b").scaled(tokens_per_rank=64, layers=2)
    ids = W.make_ids(wl).numpy()
    for p in range(ids.shape[0]):
        load, bad = oracle.histogram(ids[p], wl.num_experts)
        np.testing.assert_array_equal(load, np.bincount(ids[p], minlength=wl.num_experts))
        assert bad == 0 and load.sum() == wl.pairs_per_plan


# ---------------------------------------------------------------- reroute
def test_reroute_hand_example():
    # E = 4; expert 3 has instances at slots 2 (quota 3) and 5 (quota 1);
    # experts 0 and 1 have single instances at slots 0 and 1; expert 2 unused.
    ids = np.array([3, 1, 3, -1, 3, 0, 3, 9], np.int32)
    log2phy = np.array([[0, -1], [1, -1], [4, -1], [2, 5]], np.int32)
    logcnt = np.array([1, 1, 1, 2], np.int32)
    quota = np.array([1, 1, 3, 0, 0, 1], np.int32)
    phys, unplaced = oracle.reroute(ids, 4, quota, log2phy, logcnt)
    # the 1st..3rd pairs of expert 3 take slot 2, the 4th takes slot 5
    assert phys.tolist() == [2, 1, 2, -1, 2, 0, 5, -1]
    assert unplaced == 0


def test_reroute_short_quota_leaves_pairs_unplaced():
    ids = np.array([0, 0, 0], np.int32)
    phys, unplaced = oracle.reroute(ids, 1, np.array([2], np.int32), np.array([[0]], np.int32),
                                    np.array([1], np.int32))
    assert phys.tolist() == [0, 0, -1] and unplaced == 1


def _independent_reroute(ids, E, phy_quota, log2phy, logcnt):
    """Stable argsort by expert, then consecutive quota runs in instance order."""
    out = np.full(ids.size, -1, np.int32)
    valid = np.nonzero((ids >= 0) & (ids < E))[0]
    order = valid[np.argsort(ids[valid], kind="stable")]
    sorted_ids = ids[order]
    for e in range(E):
        pos = order[sorted_ids == e]
        inst = log2phy[e, : logcnt[e]]
        labels = np.repeat(inst, phy_quota[inst])
        assert labels.size == pos.size
        out[pos] = labels
    return out


def _check_reroute_invariants(ids, E, layout, pl, phys):
    first, home, rank, spare = layout.slots()
    valid = (ids >= 0) & (ids < E)
    assert np.all(phys[~valid] == -1)
    # (i) every pair goes to an instance of its own expert
    np.testing.assert_array_equal(pl.phy2log[phys[valid]], ids[valid])
    # (ii) every instance receives exactly its quota
    np.testing.assert_array_equal(np.bincount(phys[valid], minlength=layout.num_phys), pl.phy_quota)
    # (iii) stability: within an expert the instance index never decreases along flat order
    for e in range(E):
        p = phys[ids == e]
        if p.size:
            idx = np.searchsorted(pl.log2phy[e, : pl.logcnt[e]], p)
            assert np.all(np.diff(idx) >= 0)
    # (iv) equals the argsort construction
    np.testing.assert_array_equal(phys, _independent_reroute(ids, E, pl.phy_quota, pl.log2phy, pl.logcnt))


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_reroute_invariants_on_workloads(name):
    wl = W.get(name)
    wls = wl.scaled(tokens_per_rank=min(wl.tokens_per_rank, 48), layers=min(wl.layers, 2),
                    microbatches=min(wl.microbatches, 2))
    lay = oracle.Layout.from_workload(wl)
    ids = W.make_ids(wls).numpy()
    for p in range(ids.shape[0]):
        load, _ = oracle.histogram(ids[p], wl.num_experts)
        pl = oracle.plan(load, lay)
        phys, unplaced = oracle.reroute(ids[p], wl.num_experts, pl.phy_quota, pl.log2phy, pl.logcnt)
        assert unplaced == 0
        _check_reroute_invariants(ids[p], wl.num_experts, lay, pl, phys)


def test_reroute_identity_without_spares():
    # (v) S = 0: every pair goes to its expert's native slot
    rng = np.random.default_rng(3)
    E, R = 10, 4
    nat = np.array([3, 3, 2, 2])
    lay = oracle.Layout.of(E, R, nat, rng.permutation(E), np.zeros(R, np.int32))
    first, home, rank, _ = lay.slots()
    native_slot = np.empty(E, np.int32)
    native_slot[home[home >= 0]] = np.nonzero(home >= 0)[0]
    ids = _rand_ids(rng, 5000, E)
    load, _ = oracle.histogram(ids, E)
    pl = oracle.plan(load, lay)
    phys, _ = oracle.reroute(ids, E, pl.phy_quota, pl.log2phy, pl.logcnt)
    v = (ids >= 0) & (ids < E)
    np.testing.assert_array_equal(phys[v], native_slot[ids[v]])


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 2**31 - 1))
def test_reroute_invariants_random_layouts(seed):
    rng = np.random.default_rng(seed)
    E, R, nat, nexp, spare = W.random_layout(rng)
    lay = oracle.Layout.of(E, R, nat, nexp, spare)
    n = int(rng.integers(0, 600))
    p = rng.dirichlet(np.full(E, 0.3))
    ids = rng.choice(E, size=n, p=p).astype(np.int32)
    if n and rng.random() < 0.5:
        ids[rng.random(n) < 0.1] = -1
    load, _ = oracle.histogram(ids, E)
    pl = oracle.plan(load, lay)
    phys, unplaced = oracle.reroute(ids, E, pl.phy_quota, pl.log2phy, pl.logcnt)
    assert unplaced == 0
    _check_reroute_invariants(ids, E, lay, pl, phys)
