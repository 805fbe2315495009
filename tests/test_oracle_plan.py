"""Pins for the oracle's slot numbering, water-filling and planner (A2).

What the pages fix and is checked here:
* per-instance quotas that cover each expert's load exactly, and every
  expert keeping its native instance (UltraEP article, key designs);
* a fixed spare-slot budget per rank with no other memory (same section);
* the EPLB example's shape: 16 physical = 12 logical + 4 redundant on 8 GPUs
  with 2 slots each, four duplicated experts, no GPU holding one expert twice
  (EPLB tutorial, "12 logical + 4 redundant" example).
What the mathematics fixes: water-filling minimises the sum of squares and the
maximum of the final loads (checked by brute force over every integer split);
the greedy can never beat the exact optimum over all spare placements (brute
force with the Hall bound); special cases with closed forms.
Two planner runs traced by hand pin the step rules (hottest rank, candidate
order, re-level before replicate, lowest-index tie-breaks, the +1 remainder).
"""
import itertools
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W
from oracle.brute import brute_force_optimum, placement_optimum, slot_lower_bound

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ slot numbering
def test_layout_numbering_by_hand():
    # rank 0 natives {5,2} + 1 spare, rank 1 native {0}, rank 2 natives {4,1,3} + 2 spares
    lay = oracle.Layout.of(6, 3, [2, 1, 3], [5, 2, 0, 4, 1, 3], [1, 0, 2])
    first, home, rank, spare = lay.slots()
    assert first.tolist() == [0, 3, 4, 9]
    assert home.tolist() == [2, 5, -1, 0, 1, 3, 4, -1, -1]
    assert rank.tolist() == [0, 0, 0, 1, 2, 2, 2, 2, 2]
    assert spare.tolist() == [2, 7, 8]


def test_layout_rejects_bad_placement():
    with pytest.raises(ValueError):
        oracle.Layout.of(3, 2, [1, 1], [0, 1], [0, 0]).slots()          # expert 2 missing
    with pytest.raises(ValueError):
        oracle.Layout.of(3, 2, [2, 1], [0, 1, 1], [0, 0]).slots()       # expert 1 twice


# ------------------------------------------------------------ water-filling
def test_waterfill_by_hand():
    # T=10 over backgrounds (0, 5): level 7.5 -> loads 8 and 7, the +1 to the lower background
    assert oracle.waterfill(10, [0, 5], [0, 1]).tolist() == [8, 2]
    # the high background instance stays empty: T=3 over (0, 10)
    assert oracle.waterfill(3, [0, 10], [0, 1]).tolist() == [3, 0]
    # equal backgrounds: remainder to the lower rank first
    assert oracle.waterfill(7, [4, 4, 4], [2, 0, 1]).tolist() == [2, 3, 2]
    assert oracle.waterfill(0, [1, 2], [0, 1]).tolist() == [0, 0]


def _compositions(T, n):
    for cuts in itertools.combinations(range(T + n - 1), n - 1):
        prev, parts = -1, []
        for c in cuts + (T + n - 1,):
            parts.append(c - prev - 1)
            prev = c
        yield parts


@settings(max_examples=150, deadline=None)
@given(st.integers(0, 12), st.lists(st.integers(0, 9), min_size=1, max_size=4), st.randoms())
def test_waterfill_is_optimal_split(T, b, rnd):
    n = len(b)
    ranks = list(range(n))
    rnd.shuffle(ranks)
    q = oracle.waterfill(T, b, ranks)
    b = np.array(b)
    assert q.sum() == T and np.all(q >= 0)
    best_sq = min(sum((bi + qi) ** 2 for bi, qi in zip(b, c)) for c in _compositions(T, n))
    best_max = min(max(bi + qi for bi, qi in zip(b, c)) for c in _compositions(T, n))
    final = b + q
    assert int((final ** 2).sum()) == best_sq
    assert int(final.max()) == best_max
    # loaded instances end at one level or one below it, and no instance is left
    # two or more below the top of the loaded ones (a unit could still move down)
    filled = q > 0
    if filled.any():
        hi = final[filled].max()
        assert np.all(final[filled] >= hi - 1)
        assert np.all(final >= hi - 1)
        # the split level: the +1 goes to the smallest (background, rank) first
        keys = list(zip(b.tolist(), ranks))
        for i in np.nonzero(filled & (final == hi))[0]:
            for j in np.nonzero(final == hi - 1)[0]:
                assert keys[i] < keys[j]


# ------------------------------------------------------------ planner, by hand
def test_plan_by_hand_single_replica():
    # rank0 natives {0,1}, rank1 native {2} + 1 spare; loads (8, 4, 2)
    # step 1: hottest rank 0; expert 0 replicated to rank 1; water-fill of 8 over
    #         backgrounds (4 on rank 0, 2 on rank 1) -> level 7: quotas 3 and 5.
    # step 2: ranks tie at 7 -> rank 0; re-levelling expert 0 changes nothing and
    #         no spare is left, so the loop stops.
    lay = oracle.Layout.of(3, 2, [2, 1], [0, 1, 2], [0, 1])
    pl = oracle.plan(np.array([8, 4, 2]), lay)
    assert pl.phy2log.tolist() == [0, 1, 2, 0]
    assert pl.phy_quota.tolist() == [3, 4, 2, 5]
    assert pl.logcnt.tolist() == [2, 1, 1]
    assert pl.log2phy.tolist() == [[0, 3], [1, -1], [2, -1]]
    assert (pl.steps, pl.cap_hit) == (1, 0)


def test_plan_by_hand_relevel():
    # ranks 0,1,2 host experts 0,1,2; spares on ranks 0 and 1; loads (11, 0, 8).
    # step 1: h=0, expert 0 -> replica on rank 1 (load 0): 11 -> 6 + 5; loads (6,5,8)
    # step 2: h=2, expert 2 -> replica on rank 0 (the only free spare): backgrounds
    #         (0 on rank 2, 6 on rank 0), level 7: quotas 7 and 1; loads (7,5,7)
    # step 3: h=0 (tie with rank 2, lower index).  Candidates by quota: expert 0 (6)
    #         then expert 2 (1).  Re-level expert 0: backgrounds 1 (rank 0), 0 (rank 1)
    #         -> level 6: quotas 5 and 6; rank 0 drops to 6.  loads (6,6,7)
    # step 4: h=2; re-level of expert 2 gives 7 again, no free spare -> stop.
    lay = oracle.Layout.of(3, 3, [1, 1, 1], [0, 1, 2], [1, 1, 0])
    pl = oracle.plan(np.array([11, 0, 8]), lay)
    # slots: r0 = {0: e0, 1: spare}, r1 = {2: e1, 3: spare}, r2 = {4: e2}
    assert pl.phy2log.tolist() == [0, 2, 1, 0, 2]
    assert pl.phy_quota.tolist() == [5, 1, 0, 6, 7]
    assert pl.logcnt.tolist() == [2, 1, 2]
    assert pl.log2phy.tolist() == [[0, 3, -1], [2, -1, -1], [1, 4, -1]]
    assert (pl.steps, pl.cap_hit) == (3, 0)


def test_plan_by_hand_ties():
    # rank 0 natives {0,1}, rank 1 native {2} + spare, rank 2 native {3} + spare;
    # loads (5, 5, 0, 0).
    # step 1: h=0; candidates tie on quota 5 -> lower expert first (0).  Ranks 1
    #         and 2 tie at load 0 -> rank 1.  Water-fill of 5 over backgrounds
    #         (5 on rank 0, 0 on rank 1): all 5 to the replica.  loads (5,5,0)
    # step 2: h=0 (tie with rank 1).  Expert 0 has quota 0 on rank 0, so the only
    #         candidate is expert 1 -> replica on rank 2: 5 -> 3 (rank 0) + 2.
    #         loads (3,5,2)
    # step 3: h=1; re-level expert 0 over backgrounds (3 on rank 0, 0 on rank 1):
    #         level 4 -> quotas 1 and 4.  loads (4,4,2)
    # step 4: h=0; candidates expert 1 (3) then expert 0 (1); re-level expert 1
    #         over backgrounds (1 on rank 0, 0 on rank 2): level 3 -> 2 and 3.
    #         loads (3,4,3)
    # step 5: h=1; re-levelling expert 0 gives 4 again and no spare is free -> stop.
    lay = oracle.Layout.of(4, 3, [2, 1, 1], [0, 1, 2, 3], [0, 1, 1])
    pl = oracle.plan(np.array([5, 5, 0, 0]), lay)
    # slots: r0 = {0: e0, 1: e1}, r1 = {2: e2, 3: spare}, r2 = {4: e3, 5: spare}
    assert pl.phy2log.tolist() == [0, 1, 2, 0, 3, 1]
    assert pl.phy_quota.tolist() == [1, 2, 0, 4, 0, 3]
    assert pl.logcnt.tolist() == [2, 2, 1, 1]
    assert pl.log2phy.tolist() == [[0, 3, -1], [1, 5, -1], [2, -1, -1], [4, -1, -1]]
    assert (pl.steps, pl.cap_hit) == (4, 0)


def test_plan_by_hand_step_cap_and_spare_order():
    # ranks 0,1,2 host experts 0,1,2; spares (1, 2, 0); loads (37, 6, 34).
    # slots: r0 = {0: e0, 1: spare}, r1 = {2: e1, 3: spare, 4: spare}, r2 = {5: e2}
    # cap = 2*S + R = 2*3 + 3 = 9 moves.
    # step 1: h=0 (37).  e0 has one instance; replicate: ranks with a free spare and
    #         no e0 = {1} -> rank 1, its LOWEST free spare = slot 3.  Water-fill 37
    #         over backgrounds (0 on r0, 6 on r1): level 43/2 -> 22 and 15.
    #         loads (22, 21, 34)
    # step 2: h=2.  Replicate e2: ranks {0: 22, 1: 21} -> rank 1, next free spare =
    #         slot 4.  Water-fill 34 over (0 on r2, 21 on r1): 55/2 -> 28 and 6.
    #         loads (22, 27, 28)
    # step 3: h=2.  Re-level e2 gives 28 again; replicate e2 onto rank 0 (rank 1 is
    #         full), slot 1: 34 over (0 on r2, 21 on r1, 22 on r0): 77/3 = 25 rem 2
    #         -> 26, 5, 3.  loads (25, 26, 26); every spare is now taken.
    # step 4: h=1 (tie with r2).  Candidates e0 (15), e1 (6), e2 (5).  Re-level e0
    #         over (3 on r0, 11 on r1): 51/2 -> 23 and 14.  loads (26, 25, 26)
    # step 5: h=0.  Re-level e0 gives 23 again; e2 over (0 on r2, 20 on r1, 23 on
    #         r0): 77/3 -> 26, 6, 2.  loads (25, 26, 26)
    # step 6: h=1.  e0 over (2 on r0, 12 on r1) -> 24 and 13.  loads (26, 25, 26)
    # step 7: h=0.  e2 over (0, 19 on r1, 24 on r0) -> 26, 7, 1.  loads (25, 26, 26)
    # step 8: h=1.  e0 over (1 on r0, 13 on r1) -> 25 and 12.  loads (26, 25, 26)
    # step 9: h=0.  e2 over (0, 18 on r1, 25 on r0) -> 26, 8, 0.  loads (25, 26, 26)
    # 9 moves = the cap: the loop stops with the flag set (a tenth move, re-levelling
    # e0 on rank 1, would still lower the hottest rank).  The replica of e2 on rank 0
    # ends with quota 0 and is freed.
    lay = oracle.Layout.of(3, 3, [1, 1, 1], [0, 1, 2], [1, 2, 0])
    pl = oracle.plan(np.array([37, 6, 34]), lay)
    assert pl.phy2log.tolist() == [0, -1, 1, 0, 2, 2]
    assert pl.phy_quota.tolist() == [25, 0, 6, 12, 8, 26]
    assert pl.logcnt.tolist() == [2, 1, 2]
    assert pl.log2phy.tolist() == [[0, 3, -1], [2, -1, -1], [4, 5, -1]]
    assert (pl.steps, pl.cap_hit) == (9, 1)


def test_plan_by_hand_step_cap_with_idle_natives():
    # The same run with eight more experts (3..10) native on rank 2 and never
    # loaded: they are no candidates and change no background, so every move and
    # the cap (2*3 + 3 = 9) are as above; only rank 2's slots are renumbered
    # (5: e2, 6..13: e3..e10).
    lay = oracle.Layout.of(11, 3, [1, 1, 9], list(range(11)), [1, 2, 0])
    load = np.zeros(11, np.int64)
    load[:3] = [37, 6, 34]
    pl = oracle.plan(load, lay)
    assert pl.phy2log.tolist() == [0, -1, 1, 0, 2, 2] + list(range(3, 11))
    assert pl.phy_quota.tolist() == [25, 0, 6, 12, 8, 26] + [0] * 8
    assert pl.logcnt.tolist() == [2, 1, 2] + [1] * 8
    assert pl.log2phy.tolist()[:3] == [[0, 3, -1], [2, -1, -1], [4, 5, -1]]
    assert (pl.steps, pl.cap_hit) == (9, 1)


def test_plan_rejects_loads_outside_int32():
    # loads are counts: >= 0, and quotas and rank loads are int32 partial sums
    # of them, so a plan whose loads include a negative value or whose total
    # passes INT32_MAX makes no move: native placement, quota = load, flagged
    lay = oracle.Layout.of(3, 3, [1, 1, 1], [0, 1, 2], [1, 2, 0])
    _, home, _, _ = lay.slots()
    for load in ([37, -1, 34], [2**31 - 1, 1, 0], [2**30, 2**30, 0]):
        pl = oracle.plan(np.array(load, np.int64), lay)
        assert (pl.steps, pl.cap_hit, pl.bad_load) == (0, 0, 1)
        np.testing.assert_array_equal(pl.phy2log, home)
        np.testing.assert_array_equal(pl.phy_quota[home >= 0], np.array(load)[home[home >= 0]])
        assert pl.logcnt.tolist() == [1, 1, 1]
    # a total of exactly INT32_MAX is planned as usual
    load = np.array([2**31 - 1 - 10, 10, 0], np.int64)
    pl = oracle.plan(load, lay)
    assert pl.bad_load == 0 and pl.steps > 0
    check_plan_invariants(load, lay, pl)


# ------------------------------------------------------------ invariants
def check_plan_invariants(load, lay, pl):
    E, Phi = lay.num_experts, lay.num_phys
    first, home, rank, spare = lay.slots()
    load = np.asarray(load)
    q = pl.phy_quota.astype(np.int64)
    assert np.all(q >= 0)
    # natives keep their expert; spares hold -1 or an expert
    nat = home >= 0
    np.testing.assert_array_equal(pl.phy2log[nat], home[nat])
    assert np.all(pl.phy2log >= -1) and np.all(pl.phy2log < E)
    # empty slots carry no quota; live replicas carry some (unloaded replicas are freed)
    assert np.all(q[pl.phy2log < 0] == 0)
    assert np.all(q[(~nat) & (pl.phy2log >= 0)] > 0)
    # quotas cover each expert's load exactly
    per_e = np.zeros(E, np.int64)
    np.add.at(per_e, pl.phy2log[pl.phy2log >= 0], q[pl.phy2log >= 0])
    np.testing.assert_array_equal(per_e, load)
    # slot budget and one instance per expert per rank
    for r in range(lay.num_ranks):
        s = np.arange(first[r], first[r + 1])
        owners = pl.phy2log[s][pl.phy2log[s] >= 0]
        assert len(set(owners.tolist())) == owners.size
    # mapping tables agree with phy2log (ascending physical slots, -1 padded)
    for e in range(E):
        inst = np.nonzero(pl.phy2log == e)[0]
        assert pl.logcnt[e] == inst.size
        assert pl.log2phy[e, : inst.size].tolist() == inst.tolist()
        assert np.all(pl.log2phy[e, inst.size:] == -1)
    # never worse than the native placement
    st_ = oracle.stats(load, pl.phy_quota, lay)
    assert st_.max_after <= st_.max_before


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_plan_invariants_on_workloads(name):
    wl = W.get(name)
    wls = wl.scaled(tokens_per_rank=min(wl.tokens_per_rank, 256), layers=min(wl.layers, 3),
                    microbatches=min(wl.microbatches, 2))
    lay = oracle.Layout.from_workload(wl)
    ids = W.make_ids(wls).numpy()
    for p in range(ids.shape[0]):
        load, _ = oracle.histogram(ids[p], wl.num_experts)
        pl = oracle.plan(load, lay)
        check_plan_invariants(load, lay, pl)
        assert pl.cap_hit == 0
        pl2 = oracle.plan(load, lay)                       # deterministic
        assert pl2.phy2log.tolist() == pl.phy2log.tolist()
        assert pl2.phy_quota.tolist() == pl.phy_quota.tolist()


@settings(max_examples=120, deadline=None)
@given(st.integers(0, 2**31 - 1))
def test_plan_invariants_random_layouts(seed):
    rng = np.random.default_rng(seed)
    E, R, nat, nexp, spare = W.random_layout(rng)
    lay = oracle.Layout.of(E, R, nat, nexp, spare)
    kind = rng.integers(0, 3)
    if kind == 0:
        load = rng.integers(0, 300, size=E)
    elif kind == 1:
        load = np.zeros(E, np.int64)
        load[rng.integers(0, E)] = rng.integers(1, 1000)
    else:
        load = (rng.pareto(1.0, size=E) * 20).astype(np.int64)
    pl = oracle.plan(load, lay)
    check_plan_invariants(load, lay, pl)
    assert pl.steps <= 2 * lay.num_spare + R


# ------------------------------------------------------------ special cases
def test_uniform_load_is_identity():
    E, R = 16, 8
    lay = oracle.Layout.of(E, R, [2] * R, np.arange(E), [1] * R)
    pl = oracle.plan(np.full(E, 50), lay)
    first, home, _, _ = lay.slots()
    np.testing.assert_array_equal(pl.phy2log, home)
    assert pl.steps == 0
    assert oracle.stats(np.full(E, 50), pl.phy_quota, lay).imbalance_after == 1.0


def test_no_spares_is_identity():
    rng = np.random.default_rng(5)
    E, R = 12, 5
    lay = oracle.Layout.of(E, R, [3, 3, 2, 2, 2], rng.permutation(E), [0] * R)
    load = rng.integers(0, 1000, size=E)
    pl = oracle.plan(load, lay)
    _, home, _, _ = lay.slots()
    np.testing.assert_array_equal(pl.phy2log, home)
    np.testing.assert_array_equal(pl.phy_quota, load[home])
    assert pl.steps == 0


def test_zero_load_is_identity():
    lay = oracle.Layout.from_workload(W.get("tiny"))
    pl = oracle.plan(np.zeros(12, np.int32), lay)
    _, home, _, _ = lay.slots()
    np.testing.assert_array_equal(pl.phy2log, home)
    assert pl.phy_quota.sum() == 0 and pl.steps == 0
    st_ = oracle.stats(np.zeros(12, np.int32), pl.phy_quota, lay)
    assert st_.imbalance_before == 1.0 and st_.imbalance_after == 1.0


@pytest.mark.parametrize("Lhot", [1, 2, 5, 97, 1000, 12345])
@pytest.mark.parametrize("hot_rank", [0, 3])
def test_single_hot_expert_closed_form(Lhot, hot_rank):
    # only one expert is loaded; c ranks other than its own have a free spare:
    # the best and the greedy both spread it evenly: max load = ceil(L / (1 + c))
    E, R = 8, 6
    spare = np.array([1, 0, 2, 1, 1, 0])
    lay = oracle.Layout.of(E, R, [2, 2, 1, 1, 1, 1], np.arange(E), spare)
    first, home, rank, _ = lay.slots()
    e = int(home[first[hot_rank]])
    load = np.zeros(E, np.int64)
    load[e] = Lhot
    c = int(sum(1 for r in range(R) if r != hot_rank and spare[r] > 0))
    pl = oracle.plan(load, lay)
    st_ = oracle.stats(load, pl.phy_quota, lay)
    assert st_.max_after == -(-Lhot // (1 + c))


# ------------------------------------------------------------ optimality
def _native_rank(lay):
    first, home, rank, _ = lay.slots()
    nr = np.zeros(lay.num_experts, np.int64)
    nr[home[home >= 0]] = rank[home >= 0]
    return nr


def test_placement_optimum_by_hand():
    # two experts on one rank (loads 6 and 2), expert 0 also on rank 1:
    # X={0,1}: 8 over 2 ranks -> 4; X={1}: 2 over 1 rank -> 2; optimum 4
    assert placement_optimum([6, 2], [0b11, 0b01]) == 4
    # no replica: rank 0 carries both
    assert placement_optimum([6, 2], [0b01, 0b01]) == 8


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 2**31 - 1))
def test_greedy_never_beats_brute_force(seed):
    rng = np.random.default_rng(seed)
    E, R, nat, nexp, spare = W.random_layout(rng, max_experts=6, max_ranks=4, max_spare_per_rank=1)
    lay = oracle.Layout.of(E, R, nat, nexp, spare)
    load = rng.integers(0, 40, size=E)
    pl = oracle.plan(load, lay)
    greedy = oracle.stats(load, pl.phy_quota, lay).max_after
    opt = brute_force_optimum(load, R, _native_rank(lay), spare)
    assert greedy >= opt
    # the greedy's own placement admits at least its own max
    first, home, rank, _ = lay.slots()
    masks = [0] * E
    for s in range(lay.num_phys):
        if pl.phy2log[s] >= 0:
            masks[pl.phy2log[s]] |= 1 << int(rank[s])
    assert placement_optimum(load, masks) <= greedy
    assert slot_lower_bound(load, R, lay.num_spare) <= opt


def test_tiny_workload_gap_to_optimum():
    wl = W.get("tiny")
    lay = oracle.Layout.from_workload(wl)
    ids = W.make_ids(wl).numpy()
    gaps = []
    for p in range(ids.shape[0]):
        load, _ = oracle.histogram(ids[p], wl.num_experts)
        pl = oracle.plan(load, lay)
        greedy = oracle.stats(load, pl.phy_quota, lay).max_after
        opt = brute_force_optimum(load, wl.num_ranks, _native_rank(lay), wl.spare_count)
        assert greedy >= opt
        gaps.append((greedy, opt, int(load.sum()) / wl.num_ranks))
    print("tiny greedy/optimum/mean per plan:", gaps)


# ------------------------------------------------------------ EPLB example shape
def _golden_eplb():
    rows = []
    with open(os.path.join(GOLDEN, "eplb_example.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return np.array(rows, np.int32)


def check_eplb_shape(phy2log_row, slots_per_gpu, num_logical, num_redundant):
    row = np.asarray(phy2log_row)
    assert row.size == num_logical + num_redundant
    counts = np.bincount(row, minlength=num_logical)
    assert counts.size == num_logical and np.all(counts >= 1)
    assert int((counts - 1).sum()) == num_redundant
    for g in range(row.size // slots_per_gpu):
        gpu = row[g * slots_per_gpu:(g + 1) * slots_per_gpu]
        assert len(set(gpu.tolist())) == gpu.size
    return set(np.nonzero(counts > 1)[0].tolist())


def test_eplb_golden_table_shape():
    t = _golden_eplb()
    assert t.shape == (2, 16)
    dup0 = check_eplb_shape(t[0], 2, 12, 4)
    assert dup0 == {5, 4, 10, 1}
    check_eplb_shape(t[1], 2, 12, 4)
    assert not np.array_equal(t[0], t[1])


def test_reroute_on_eplb_placement():
    # EPLB's layer-0 table as a placement: the logical expert 5 lives in
    # physical slots 0 and 2; its first quota[0] pairs go to slot 0, the rest to 2
    row = _golden_eplb()[0]
    E, rho = 12, 2
    logcnt = np.bincount(row, minlength=E).astype(np.int32)
    log2phy = np.full((E, rho), -1, np.int32)
    for e in range(E):
        s = np.nonzero(row == e)[0]
        log2phy[e, : s.size] = s
    assert log2phy[5].tolist() == [0, 2] and log2phy[1].tolist() == [13, 15]
    quota = np.zeros(16, np.int32)
    ids = np.array([5, 1, 5, 5, 1, 7, 5], np.int32)
    load = np.bincount(ids, minlength=E)
    for e in range(E):                       # first instance takes ceil(half)
        s = log2phy[e, : logcnt[e]]
        quota[s[0]] = load[e] - load[e] // 2 if s.size == 2 else load[e]
        if s.size == 2:
            quota[s[1]] = load[e] // 2
    phys, unplaced = oracle.reroute(ids, E, quota, log2phy, logcnt)
    assert phys.tolist() == [0, 13, 0, 2, 15, 3, 2] and unplaced == 0


def test_tiny_plan_matches_eplb_example_shape():
    # on the 8-GPU, 2-slots-per-GPU layout, a plan that uses all four spare slots
    # has the EPLB example's shape: 12 distinct experts, four of them twice
    wl = W.get("tiny")
    lay = oracle.Layout.from_workload(wl)
    ids = W.make_ids(wl).numpy()
    seen_full = 0
    for p in range(ids.shape[0]):
        load, _ = oracle.histogram(ids[p], wl.num_experts)
        pl = oracle.plan(load, lay)
        if np.all(pl.phy2log >= 0):
            check_eplb_shape(pl.phy2log, 2, 12, 4)
            seen_full += 1
    assert seen_full >= 1
