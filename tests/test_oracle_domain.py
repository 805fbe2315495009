"""Pins for the domain-constrained planner (next row).

Hot-expert replication stays inside the high-bandwidth scale-up domain
(UltraEP article, section on why it reaches the optimum); on MI355X a domain
is one 8-GPU xGMI node.  With D ranks per domain, a replica of expert e may
only sit on a rank r with r // D == native_rank(e) // D.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W
from oracle.brute import brute_force_optimum
from test_oracle_plan import check_plan_invariants


def test_domain_by_hand():
    # ranks 0..3 host experts 0..3; spares on ranks 1 and 2; loads (12, 5, 0, 0)
    # free placement: expert 0 -> rank 2 (idle), 12 -> 6 + 6
    # domains {0,1}, {2,3}: only rank 1's spare is in expert 0's domain:
    #   backgrounds 0 (rank 0) and 5 (rank 1), level 8.5 -> quotas 9 and 3
    lay = oracle.Layout.of(4, 4, [1, 1, 1, 1], [0, 1, 2, 3], [0, 1, 1, 0])
    free = oracle.plan(np.array([12, 5, 0, 0]), lay, 0)
    assert free.phy2log.tolist() == [0, 1, -1, 2, 0, 3] and free.phy_quota.tolist() == [6, 5, 0, 0, 6, 0]
    dom = oracle.plan(np.array([12, 5, 0, 0]), lay, 2)
    assert dom.phy2log.tolist() == [0, 1, 0, 2, -1, 3] and dom.phy_quota.tolist() == [9, 5, 3, 0, 0, 0]
    assert dom.steps == 1


@pytest.mark.parametrize("name", ["tiny", "qwen3_235b", "deepseek_v3", "glm_4_5"])
def test_domain_invariants_and_limits(name):
    wl = W.get(name)
    wls = wl.scaled(tokens_per_rank=min(wl.tokens_per_rank, 200), layers=2)
    lay = oracle.Layout.from_workload(wl)
    first, home, rank, spare = lay.slots()
    native_rank = np.zeros(wl.num_experts, np.int64)
    native_rank[home[home >= 0]] = rank[home >= 0]
    ids = W.make_ids(wls).numpy()
    for p in range(ids.shape[0]):
        load, _ = oracle.histogram(ids[p], wl.num_experts)
        for D in (1, 2, 8, wl.num_ranks):
            pl = oracle.plan(load, lay, D)
            check_plan_invariants(load, lay, pl)
            for s in spare:
                e = pl.phy2log[s]
                if e >= 0:
                    assert rank[s] // D == native_rank[e] // D
        # one domain = no constraint; one rank per domain = no replica
        np.testing.assert_array_equal(oracle.plan(load, lay, wl.num_ranks).phy2log, oracle.plan(load, lay, 0).phy2log)
        np.testing.assert_array_equal(oracle.plan(load, lay, 1).phy2log, home)
        # a tighter domain never balances better than a looser one on these loads
        m = [oracle.stats(load, oracle.plan(load, lay, D).phy_quota, lay).max_after for D in (1, wl.num_ranks)]
        assert m[0] >= m[1]


@settings(max_examples=30, deadline=None)
@given(st.integers(0, 2**31 - 1))
def test_domain_greedy_never_beats_constrained_optimum(seed):
    rng = np.random.default_rng(seed)
    E, R, nat, nexp, spare = W.random_layout(rng, max_experts=6, max_ranks=4, max_spare_per_rank=1)
    D = int(rng.integers(1, R + 1))
    lay = oracle.Layout.of(E, R, nat, nexp, spare)
    first, home, rank, _ = lay.slots()
    native_rank = np.zeros(E, np.int64)
    native_rank[home[home >= 0]] = rank[home >= 0]
    load = rng.integers(0, 40, size=E)
    pl = oracle.plan(load, lay, D)
    greedy = oracle.stats(load, pl.phy_quota, lay).max_after
    assert greedy >= brute_force_optimum(load, R, native_rank, spare, ranks_per_domain=D)
