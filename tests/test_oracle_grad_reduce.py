"""Pins for the oracle's replica gradient reduction (next row).

Each replicated expert's gradient becomes the fp32 fold of its instances'
gradients in ascending physical-slot order (UltraEP article, key designs and
backward paragraph: replica gradients are reduced back to the native expert
with a fixed accumulation order, so the result is deterministic).
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _plan_for(lay, load):
    return oracle.plan(np.asarray(load, np.int32), lay)


def test_fold_order_by_hand():
    # expert 0 native on rank 1 (slot 2); replicas in the spare slots of rank 0
    # (slot 1, spare ordinal 0) and rank 2 (slot 4, spare ordinal 1).
    # Slot order of its instances: 1 (replica), 2 (native), 4 (replica).
    lay = oracle.Layout.of(3, 3, [1, 1, 1], [1, 0, 2], [1, 0, 1])
    first, home, rank, spare = lay.slots()
    assert home.tolist() == [1, -1, 0, 2, -1] and spare.tolist() == [1, 4]
    log2phy = np.array([[1, 2, 4], [0, -1, -1], [3, -1, -1]], np.int32)
    logcnt = np.array([3, 1, 1], np.int32)
    native = np.array([[1.0, 3.0], [7.0, 7.0], [9.0, 9.0]], np.float32)    # rows = experts 0, 1, 2
    slot = np.array([[1e8, 2.0], [-1e8, 5.0]], np.float32)                  # spare ordinals 0, 1
    oracle.grad_reduce(native, slot, lay, log2phy, logcnt)
    # fp32: (1e8 + 1) rounds to 1e8 (the spacing of fp32 there is 8), minus 1e8 = 0
    assert native[0].tolist() == [0.0, 10.0]
    assert native[1].tolist() == [7.0, 7.0] and native[2].tolist() == [9.0, 9.0]
    assert slot.tolist() == [[1e8, 2.0], [-1e8, 5.0]]


@pytest.mark.parametrize("name", ["tiny", "qwen3_235b", "stress"])
def test_integer_gradients_sum_exactly(name):
    wl = W.get(name)
    lay = oracle.Layout.from_workload(wl)
    ids = W.make_ids(wl.scaled(tokens_per_rank=min(wl.tokens_per_rank, 64), layers=1, microbatches=1)).numpy()
    pl = _plan_for(lay, oracle.histogram(ids[0], wl.num_experts)[0])
    rng = np.random.default_rng(1)
    n = 24
    native = rng.integers(-1000, 1000, size=(wl.num_experts, n)).astype(np.float32)
    slot = rng.integers(-1000, 1000, size=(lay.num_spare, n)).astype(np.float32)
    before = native.copy()
    first, home, rank, spare = lay.slots()
    spare_of = {int(s): o for o, s in enumerate(spare)}
    oracle.grad_reduce(native, slot, lay, pl.log2phy, pl.logcnt)
    for e in range(wl.num_experts):
        inst = pl.log2phy[e, : pl.logcnt[e]]
        if inst.size < 2:
            np.testing.assert_array_equal(native[e], before[e])
            continue
        exp = np.zeros(n, np.float64)
        for s in inst:
            exp += before[e] if home[s] >= 0 else slot[spare_of[int(s)]]
        np.testing.assert_array_equal(native[e].astype(np.float64), exp)


def test_error_within_fp32_bound():
    wl = W.get("stress")
    lay = oracle.Layout.from_workload(wl)
    ids = W.make_ids(wl.scaled(tokens_per_rank=64, layers=1, microbatches=1)).numpy()
    pl = _plan_for(lay, oracle.histogram(ids[0], wl.num_experts)[0])
    rng = np.random.default_rng(2)
    n = 64
    native = rng.standard_normal((wl.num_experts, n)).astype(np.float32)
    slot = rng.standard_normal((lay.num_spare, n)).astype(np.float32)
    before = native.astype(np.float64)
    first, home, rank, spare = lay.slots()
    spare_of = {int(s): o for o, s in enumerate(spare)}
    oracle.grad_reduce(native, slot, lay, pl.log2phy, pl.logcnt)
    eps = np.finfo(np.float32).eps / 2
    for e in range(wl.num_experts):
        inst = pl.log2phy[e, : pl.logcnt[e]]
        if inst.size < 2:
            continue
        terms = np.stack([before[e] if home[s] >= 0 else slot[spare_of[int(s)]].astype(np.float64) for s in inst])
        exact = terms.sum(axis=0)
        bound = (inst.size - 1) * eps * np.abs(terms).sum(axis=0) * 1.0001
        assert np.all(np.abs(native[e] - exact) <= bound)
