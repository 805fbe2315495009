"""Pins for the oracle's dispatch layout (next row after the reroute).

The dispatch order is the pairs sorted by physical slot, stable in flat order
(EPLB tutorial, EPLB / DeepEP section: dispatch sends by physical replica,
combine gathers back); with quotas that cover every expert's load this is a
plain stable counting sort, so it is checked against numpy's stable argsort,
and slot offsets against the bincount prefix.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def test_dispatch_hand_example():
    # expert 3 has instances at slots 2 (quota 3) and 5 (quota 1); experts 0, 1
    # at slots 0, 1 (quota 1 each); Phi = 6, slot 3 and 4 empty
    ids = np.array([3, 1, 3, -1, 3, 0, 3], np.int32)
    log2phy = np.array([[0, -1], [1, -1], [4, -1], [2, 5]], np.int32)
    logcnt = np.array([1, 1, 1, 2], np.int32)
    quota = np.array([1, 1, 3, 0, 0, 1], np.int32)
    off, pos, src, placed = oracle.dispatch(ids, 4, quota, log2phy, logcnt)
    assert off.tolist() == [0, 1, 2, 5, 5, 5, 6]
    # slot 0: pair 5; slot 1: pair 1; slot 2: pairs 0, 2, 4; slot 5: pair 6
    assert src.tolist() == [5, 1, 0, 2, 4, 6, -1]
    assert pos.tolist() == [2, 1, 3, -1, 4, 0, 5]
    assert placed == 6


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_dispatch_is_stable_sort_by_slot(name):
    wl = W.get(name)
    wls = wl.scaled(tokens_per_rank=min(wl.tokens_per_rank, 40), layers=2, microbatches=1)
    lay = oracle.Layout.from_workload(wl)
    ids = W.inject_invalid(W.make_ids(wls), wl.num_experts, 0.03, 0.01).numpy()
    for p in range(ids.shape[0]):
        load, _ = oracle.histogram(ids[p], wl.num_experts)
        pl = oracle.plan(load, lay)
        phys, _ = oracle.reroute(ids[p], wl.num_experts, pl.phy_quota, pl.log2phy, pl.logcnt)
        off, pos, src, placed = oracle.dispatch(ids[p], wl.num_experts, pl.phy_quota, pl.log2phy, pl.logcnt)
        valid = np.nonzero(phys >= 0)[0]
        order = valid[np.argsort(phys[valid], kind="stable")]
        assert placed == valid.size
        np.testing.assert_array_equal(src[: valid.size], order)
        assert np.all(src[valid.size:] == -1)
        np.testing.assert_array_equal(pos[order], np.arange(valid.size))
        assert np.all(pos[phys < 0] == -1)
        cnt = np.bincount(phys[valid], minlength=lay.num_phys)
        np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(cnt)]))
        # each slot's pairs form one block in the order
        assert np.all(np.diff(phys[src[: valid.size]]) >= 0)
