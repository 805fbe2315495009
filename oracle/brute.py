"""Exact optimum and lower bound for the replica-placement problem (test infrastructure).

The problem, as the UltraEP article states it (section on the key designs):
every rank owns a fixed number of spare slots that may hold copies of hot
experts, and the load (token count) of each expert is split into per-instance
quotas; the aim is the smallest possible load on the most loaded rank.

For one fixed placement, the smallest achievable maximum is a transportation
problem: expert e ships load[e] units to the ranks hosting one of its
instances, and every rank takes at most lam units.  By the supply-demand
(Gale / Hall) theorem lam is feasible iff for every set X of experts
load(X) <= lam * |N(X)|, where N(X) is the set of ranks hosting any instance
of an expert in X; since max-flow has integral solutions, the integer optimum
is max over X of ceil(load(X) / |N(X)|).  Enumerating every placement of the
spare slots (each spare slot empty or holding any expert not already on its
rank) gives the exact optimum for tiny instances.
"""
from __future__ import annotations

import itertools
from typing import Sequence

import numpy as np


def placement_optimum(load: Sequence[int], expert_ranks: Sequence[int]) -> int:
    """min over integer quotas of the max rank load; expert_ranks[e] = bitmask of ranks hosting e."""
    load = np.asarray(load, dtype=np.int64)
    E = load.size
    subsets = np.arange(1, 1 << E, dtype=np.int64)
    lx = np.zeros(subsets.size, np.int64)
    nx = np.zeros(subsets.size, np.int64)
    for e in range(E):
        sel = (subsets >> e) & 1
        lx += sel * load[e]
        nx |= sel * int(expert_ranks[e])
    cnt = np.array([bin(int(m)).count("1") for m in nx], np.int64)
    return int(np.max(-(-lx // cnt))) if subsets.size else 0


def _popcount_vec(x: np.ndarray) -> np.ndarray:
    c = np.zeros_like(x)
    y = x.copy()
    while np.any(y):
        c += y & 1
        y >>= 1
    return c


def brute_force_optimum(load: Sequence[int], num_ranks: int, native_rank: Sequence[int],
                        spare_count: Sequence[int], ranks_per_domain: int = 0) -> int:
    """Exact minimum of the max rank load over every use of the spare slots.

    ``native_rank[e]`` is the rank hosting expert e's native instance.  A spare
    slot is empty or holds one expert that its rank does not host yet (a second
    instance on one rank never lowers that rank's load).
    """
    load = np.asarray(load, dtype=np.int64)
    E = load.size
    R = num_ranks
    base_mask = np.array([1 << int(native_rank[e]) for e in range(E)], np.int64)
    subsets = np.arange(1, 1 << E, dtype=np.int64)
    sel = ((subsets[:, None] >> np.arange(E)[None, :]) & 1).astype(np.int64)   # [X][E]
    lx = sel @ load
    native_nx = np.zeros(subsets.size, np.int64)
    for e in range(E):
        native_nx |= sel[:, e] * int(base_mask[e])
    hosted = [set(int(e) for e in range(E) if native_rank[e] == r) for r in range(R)]

    # choices per rank: tuples of distinct experts not native on r (order-free), size <= spare
    per_rank = []
    for r in range(R):
        pool = [e for e in range(E) if e not in hosted[r] and
                (ranks_per_domain <= 0 or r // ranks_per_domain == int(native_rank[e]) // ranks_per_domain)]
        opts = []
        for k in range(0, int(spare_count[r]) + 1):
            opts.extend(itertools.combinations(pool, k))
        per_rank.append(opts)

    best = None
    for choice in itertools.product(*per_rank):
        nx = native_nx.copy()
        for r, exps in enumerate(choice):
            for e in exps:
                nx |= sel[:, e] * (1 << r)
        lam = int(np.max(-(-lx // _popcount_vec(nx))))
        if best is None or lam < best:
            best = lam
    return int(best if best is not None else 0)


def slot_lower_bound(load: Sequence[int], num_ranks: int, num_spare: int) -> int:
    """Smallest lam >= ceil(total/R) with sum_e (ceil(load_e/lam) - 1) <= S.

    Any plan with maximum rank load lam gives each instance at most lam units
    and puts the instances of one expert on distinct ranks, so expert e needs at
    least ceil(load_e/lam) instances, i.e. that many minus one spare slots.
    """
    load = np.asarray(load, dtype=np.int64)
    total = int(load.sum())
    if total == 0:
        return 0
    lo = max(-(-total // num_ranks), 1)
    hi = max(int(load.max()), lo)

    def ok(lam: int) -> bool:
        extra = np.maximum(-(-load // lam) - 1, 0)    # an unloaded expert needs no copy
        return int(np.sum(extra)) <= num_spare

    while lo < hi:
        mid = (lo + hi) // 2
        if ok(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


def milp_bounds(load: Sequence[int], num_ranks: int, native_rank: Sequence[int],
                spare_count: Sequence[int], time_limit: float = 30.0):
    """Bounds on the optimum of the same problem at sizes brute force cannot reach.

    A mixed-integer program: x[e][r] in {0, 1} says that a spare slot of rank r
    holds a copy of expert e (never on e's native rank); q[e][r] >= 0 is the
    load expert e sends to rank r (its native rank, or a rank holding a copy:
    q[e][r] <= load[e] * x[e][r]); the quotas of e add up to load[e]; rank r
    holds at most spare_count[r] copies and takes at most lam in all; minimise
    lam.  For one placement the best quotas form a transportation problem whose
    integer optimum is the ceiling of its fractional one, so the integer optimum
    over placements is ceil(lam*).  Solved by HiGHS (scipy.optimize.milp) within
    ``time_limit`` seconds; returns (status, best lam found or None, proven lower
    bound on lam*), status 0 when lam* is proven optimal.
    """
    from scipy.optimize import Bounds, LinearConstraint, milp
    from scipy.sparse import csr_matrix

    load = np.asarray(load, dtype=np.int64)
    E, R = load.size, int(num_ranks)
    spare_ranks = [r for r in range(R) if int(spare_count[r]) > 0]
    copies = [(e, r) for e in range(E) for r in spare_ranks if int(native_rank[e]) != r and load[e] > 0]
    nc = len(copies)
    # variables: x[0..nc), q_native[e] at nc + e, q_copy[k] at nc + E + k, lam last
    n = nc + E + nc + 1
    lam = n - 1
    rows, cols, vals, lo, hi = [], [], [], [], []

    def row(entries, low, high):
        r = len(lo)
        for c, v in entries:
            rows.append(r); cols.append(c); vals.append(v)
        lo.append(low); hi.append(high)

    by_expert = [[] for _ in range(E)]
    by_rank = {r: [] for r in spare_ranks}
    for k, (e, r) in enumerate(copies):
        by_expert[e].append(k)
        by_rank[r].append(k)
    for e in range(E):
        row([(nc + e, 1.0)] + [(nc + E + k, 1.0) for k in by_expert[e]], float(load[e]), float(load[e]))
    for k, (e, r) in enumerate(copies):
        row([(nc + E + k, 1.0), (k, -float(load[e]))], -np.inf, 0.0)
    for r in spare_ranks:
        row([(k, 1.0) for k in by_rank[r]], -np.inf, float(spare_count[r]))
    for r in range(R):
        entries = [(nc + e, 1.0) for e in range(E) if int(native_rank[e]) == r]
        entries += [(nc + E + k, 1.0) for k in by_rank.get(r, [])]
        row(entries + [(lam, -1.0)], -np.inf, 0.0)
    A = csr_matrix((vals, (rows, cols)), shape=(len(lo), n))
    c = np.zeros(n)
    c[lam] = 1.0
    integrality = np.zeros(n)
    integrality[:nc] = 1
    upper = np.concatenate([np.ones(nc), np.full(E + nc + 1, np.inf)])
    res = milp(c, constraints=LinearConstraint(A, lo, hi), integrality=integrality,
               bounds=Bounds(np.zeros(n), upper), options={"time_limit": float(time_limit)})
    best = float(res.fun) if res.fun is not None else None
    bound = getattr(res, "mip_dual_bound", None)
    bound = float(bound) if bound is not None else (best if res.status == 0 else 0.0)
    return int(res.status), best, bound
