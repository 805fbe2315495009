"""Pins for the oracle's balance statistics (A5) and slot fill (A4).

Imbalance is the most loaded rank over the mean rank load (UltraEP digest,
"Reported results"); EPLB's balancedness is its reciprocal (EPLB tutorial,
measured-speedup section).  The slot fill is a pure copy of the chosen
experts' weights into the reserved, layer-shared slot buffer (UltraEP
article, key designs), so it is checked against numpy's take.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def test_stats_by_hand():
    # plan of the hand-traced case: ranks host experts 0,1,2; loads (11,0,8)
    lay = oracle.Layout.of(3, 3, [1, 1, 1], [0, 1, 2], [1, 1, 0])
    load = np.array([11, 0, 8])
    quota = np.array([5, 1, 0, 6, 7])          # slots r0{e0, spare}, r1{e1, spare}, r2{e2}
    st = oracle.stats(load, quota, lay)
    assert st.rank_before.tolist() == [11, 0, 8]
    assert st.rank_after.tolist() == [6, 6, 7]
    assert (st.max_before, st.max_after, st.total, st.replicas_used) == (11, 7, 19, 2)
    assert st.imbalance_before == 11 * 3 / 19
    assert st.imbalance_after == 7 * 3 / 19


@pytest.mark.parametrize("name", ["tiny", "qwen3_235b", "glm_4_5"])
def test_stats_recomputed_from_rerouted_pairs(name):
    wl = W.get(name)
    wls = wl.scaled(tokens_per_rank=min(wl.tokens_per_rank, 64), layers=2)
    lay = oracle.Layout.from_workload(wl)
    first, home, rank, spare = lay.slots()
    ids = W.make_ids(wls).numpy()
    for p in range(ids.shape[0]):
        load, _ = oracle.histogram(ids[p], wl.num_experts)
        pl = oracle.plan(load, lay)
        phys, _ = oracle.reroute(ids[p], wl.num_experts, pl.phy_quota, pl.log2phy, pl.logcnt)
        st = oracle.stats(load, pl.phy_quota, lay)
        # after: count the rerouted pairs landing on each rank
        after = np.bincount(rank[phys[phys >= 0]], minlength=wl.num_ranks)
        np.testing.assert_array_equal(st.rank_after, after)
        # before: count the pairs whose expert is native on each rank
        native_rank = np.zeros(wl.num_experts, np.int64)
        native_rank[home[home >= 0]] = rank[home >= 0]
        before = np.bincount(native_rank[ids[p]], minlength=wl.num_ranks)
        np.testing.assert_array_equal(st.rank_before, before)
        assert st.total == ids[p].size
        assert st.imbalance_after == float(after.max() * wl.num_ranks) / float(ids[p].size)
        assert st.replicas_used == int(np.sum(pl.phy2log[spare] >= 0))
        assert st.imbalance_after <= st.imbalance_before


def test_slot_fill_matches_take():
    wl = W.get("tiny")
    lay = oracle.Layout.from_workload(wl)
    first, home, rank, spare = lay.slots()
    w = W.make_weights(wl).view(__import__("torch").int16).numpy()     # bf16 bits
    ids = W.make_ids(wl).numpy()
    for p in range(ids.shape[0]):
        load, _ = oracle.histogram(ids[p], wl.num_experts)
        pl = oracle.plan(load, lay)
        buf = np.full((lay.num_spare, w.shape[1]), 0x7FC1, np.int16)   # sentinel
        oracle.slot_fill(w, pl.phy2log, lay, buf)
        for o, s in enumerate(spare):
            e = pl.phy2log[s]
            if e >= 0:
                np.testing.assert_array_equal(buf[o], np.take(w, e, axis=0))
            else:
                assert np.all(buf[o] == 0x7FC1)


def test_slot_fill_leaves_empty_slots():
    lay = oracle.Layout.of(3, 2, [2, 1], [0, 1, 2], [1, 2])
    w = np.arange(3 * 8, dtype=np.uint8).reshape(3, 8)
    buf = np.full((3, 8), 0xEE, np.uint8)
    phy2log = np.array([0, 1, -1, 2, 0, -1], np.int32)   # r0{0,1,spare} r1{2,spare,spare}
    oracle.slot_fill(w, phy2log, lay, buf)
    assert buf[0].tolist() == [0xEE] * 8
    assert buf[1].tolist() == w[0].tolist()
    assert buf[2].tolist() == [0xEE] * 8


def test_slot_fill_entries_that_name_no_expert_are_empty():
    # a phy2log entry outside [0, E) names no expert: that spare slot is empty
    lay = oracle.Layout.of(3, 2, [2, 1], [0, 1, 2], [1, 2])
    w = np.arange(3 * 8, dtype=np.uint8).reshape(3, 8)
    buf = np.full((3, 8), 0xEE, np.uint8)
    phy2log = np.array([0, 1, 3, 2, 2, 2 ** 31 - 1], np.int32)  # spares: E, expert 2, INT32_MAX
    oracle.slot_fill(w, phy2log, lay, buf)
    assert buf[0].tolist() == [0xEE] * 8
    assert buf[1].tolist() == w[2].tolist()
    assert buf[2].tolist() == [0xEE] * 8
