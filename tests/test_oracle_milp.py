"""The placement problem at scale: MILP bounds pinned to brute force, and the
greedy planner's gap to them on the DeepSeek-V3-like workload.

The MILP (oracle.brute.milp_bounds) is pinned against the exhaustive optimum on
tiny instances; on full-size plans it gives a proven lower bound on the optimum
(and usually a better placement than the greedy's), which measures how far the
greedy reading of the solver stays from optimal where the slot-count bound is
loose.  EP_MILP_SECONDS (default 20) sets the solver's time per plan and
EP_MILP_PLANS (default "0") the plans; run with -s to see the numbers.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as W
from oracle.brute import brute_force_optimum, milp_bounds, slot_lower_bound

pytest.importorskip("scipy.optimize")


@pytest.mark.parametrize("seed", range(6))
def test_milp_optimum_equals_brute_force_on_tiny(seed):
    rng = np.random.default_rng(1000 + seed)
    E, R = int(rng.integers(3, 6)), int(rng.integers(2, 4))
    native_rank = sorted(int(x) for x in rng.integers(0, R, E))
    spare = [int(x) for x in rng.integers(0, 2, R)]
    load = [int(x) for x in rng.integers(0, 40, E)]
    exact = brute_force_optimum(load, R, native_rank, spare)
    status, best, bound = milp_bounds(load, R, native_rank, spare, time_limit=30)
    assert status == 0
    assert int(np.ceil(best - 1e-6)) == exact, (load, native_rank, spare)
    assert bound <= best + 1e-6


def test_greedy_gap_at_scale_deepseek_v3():
    wl = W.get("deepseek_v3")
    lay = oracle.Layout.from_workload(wl)
    native_rank = [r for r, n in enumerate(wl.native_count) for _ in range(n)]
    secs = float(os.environ.get("EP_MILP_SECONDS", "20"))
    plans = [int(p) for p in os.environ.get("EP_MILP_PLANS", "0").split(",")]
    ids = W.make_ids(wl, device="cpu", plans=plans).numpy()
    for i, p in enumerate(plans):
        load = oracle.histogram(ids[i], wl.num_experts)[0]
        greedy = int(oracle.stats(load, oracle.plan(load, lay).phy_quota, lay).as_row()[1])
        mean = load.sum() / wl.num_ranks
        slot = slot_lower_bound(load, wl.num_ranks, wl.num_spare)
        status, best, bound = milp_bounds(load, wl.num_ranks, native_rank, wl.spare_count, time_limit=secs)
        # the greedy's placement is feasible, so nothing proven below the optimum exceeds it
        assert bound <= greedy + 1e-6
        assert slot <= greedy
        print(f"\n[deepseek_v3 plan {p}] max rank load / mean: greedy {greedy / mean:.3f}, "
              f"MILP best {best / mean if best else float('nan'):.3f}, proven optimum >= "
              f"{max(bound, slot) / mean:.3f} (slot-count bound {slot / mean:.3f}; {secs:.0f} s, status {status})")
