"""GPU parity: every step of the HIP path against the CPU oracle, bit-exact.

Each kernel is first fed the oracle's own inputs (the planner gets the
oracle's loads, the reroute the oracle's plan tables, the slot fill the
oracle's phy2log), then the full chain runs on the GPU alone.  Tolerance is 0
everywhere: the work is integer (plus one correctly rounded double division
in the statistics) and a pure copy.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

ep = pytest.importorskip("moe_expert_load_layer_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _small(name, tokens=37, layers=3, mbs=1):
    wl = W.get(name)
    return wl, wl.scaled(tokens_per_rank=min(tokens, wl.tokens_per_rank), layers=min(layers, wl.layers),
                         microbatches=min(mbs, wl.microbatches))


def _np(t):
    return t.detach().cpu().numpy()


def _stack_plans(plans):
    return (np.stack([p.phy2log for p in plans]), np.stack([p.phy_quota for p in plans]),
            np.stack([p.logcnt for p in plans]), np.stack([p.log2phy for p in plans]),
            np.array([p.steps for p in plans]))


def _assert_plan_equal(gpu_plan, ref_plans):
    p2l, q, lc, l2p, steps = _stack_plans(ref_plans)
    np.testing.assert_array_equal(_np(gpu_plan.phy2log), p2l)
    np.testing.assert_array_equal(_np(gpu_plan.phy_quota), q)
    np.testing.assert_array_equal(_np(gpu_plan.logcnt), lc)
    np.testing.assert_array_equal(_np(gpu_plan.log2phy), l2p)
    np.testing.assert_array_equal(_np(gpu_plan.steps), steps)


# --------------------------------------------------------------------- A1
@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_histogram_matches_oracle(dev, name):
    wl, wls = _small(name)
    ids = W.make_ids(wls)
    print(f"[hist] {name} P={ids.shape[0]} N={ids.shape[1]}", flush=True)
    lay = ep.Layout.from_workload(wl, device=dev)
    load, ws, status = ep.ep_load_histogram(ids.to(dev), lay)
    torch.cuda.synchronize()
    for p in range(ids.shape[0]):
        ref, bad = oracle.histogram(ids[p].numpy(), wl.num_experts)
        np.testing.assert_array_equal(_np(load[p]), ref)
        assert int(status[p]) == 0 and bad == 0


@pytest.mark.parametrize("N", [0, 1, 3, 63, 64, 65, 2047, 2048, 2049, 6151, 20001])
def test_histogram_sizes_padding_and_bad_ids(dev, N):
    rng = np.random.default_rng(N)
    E, P = 19, 3
    ids = torch.from_numpy(rng.integers(0, E, size=(P, N)).astype(np.int32))
    ids = W.inject_invalid(ids, E, 0.07, 0.03, seed=N) if N else ids
    print(f"[hist-sizes] N={N}", flush=True)
    lay = ep.Layout.create(E, [5, 5, 5, 4], list(range(E)), [1, 0, 2, 1], device=dev)
    load, ws, status = ep.ep_load_histogram(ids.to(dev), lay)
    torch.cuda.synchronize()
    for p in range(P):
        ref, bad = oracle.histogram(ids[p].numpy(), E)
        np.testing.assert_array_equal(_np(load[p]), ref)
        assert int(status[p]) == (ep.EP_STATUS_BAD_ID if bad else 0)


# --------------------------------------------------------------------- A2
@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_plan_matches_oracle(dev, name):
    wl, wls = _small(name, tokens=200, layers=4, mbs=2)
    lay_o = oracle.Layout.from_workload(wl)
    ids = W.make_ids(wls).numpy()
    loads = np.stack([oracle.histogram(ids[p], wl.num_experts)[0] for p in range(ids.shape[0])])
    refs = [oracle.plan(l, lay_o) for l in loads]
    print(f"[plan] {name} P={loads.shape[0]} steps={[r.steps for r in refs]}", flush=True)
    lay = ep.Layout.from_workload(wl, device=dev)
    status = torch.zeros(loads.shape[0], dtype=torch.int32, device=dev)
    out = ep.ep_plan_quota(torch.from_numpy(loads).to(dev), lay, status=status)
    torch.cuda.synchronize()
    _assert_plan_equal(out, refs)
    np.testing.assert_array_equal(_np(status), [ep.EP_STATUS_STEP_CAP if r.cap_hit else 0 for r in refs])


def test_plan_hand_cases(dev):
    cases = [
        (3, [2, 1], [0, 1, 2], [0, 1], [8, 4, 2]),
        (3, [1, 1, 1], [0, 1, 2], [1, 1, 0], [11, 0, 8]),
        (4, [2, 1, 1], [0, 1, 2, 3], [0, 1, 1], [5, 5, 0, 0]),
    ]
    for E, nc, ne, sc, load in cases:
        lay_o = oracle.Layout.of(E, len(nc), nc, ne, sc)
        ref = oracle.plan(np.array(load), lay_o)
        lay = ep.Layout.create(E, nc, ne, sc, device=dev)
        out = ep.ep_plan_quota(torch.tensor([load], dtype=torch.int32, device=dev), lay)
        torch.cuda.synchronize()
        _assert_plan_equal(out, [ref])


@pytest.mark.parametrize("seed", range(6))
def test_plan_random_layouts(dev, seed):
    rng = np.random.default_rng(1000 + seed)
    for it in range(8):
        E, R, nc, ne, sc = W.random_layout(rng, max_experts=70, max_ranks=40, max_spare_per_rank=3)
        lay_o = oracle.Layout.of(E, R, nc, ne, sc)
        if lay_o.max_replicas > 64:
            continue
        P = int(rng.integers(1, 5))
        kind = it % 3
        if kind == 0:
            loads = rng.integers(0, 3000, size=(P, E))
        elif kind == 1:
            loads = (rng.pareto(0.8, size=(P, E)) * 50).astype(np.int64)
        else:
            loads = np.zeros((P, E), np.int64)
            loads[:, rng.integers(0, E)] = rng.integers(1, 10**6)
        loads = loads.astype(np.int32)
        refs = [oracle.plan(l, lay_o) for l in loads]
        lay = ep.Layout.create(E, nc, ne, sc, device=dev)
        out = ep.ep_plan_quota(torch.from_numpy(loads).to(dev), lay)
        torch.cuda.synchronize()
        _assert_plan_equal(out, refs)


def test_plan_max_replicas_64(dev):
    # rho = 64: 64 ranks with 2 spares each; one expert carries most of the load
    E, R = 64, 64
    nc, ne, sc = [1] * R, list(range(E)), [2] * R
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    assert lay_o.max_replicas == 64
    rng = np.random.default_rng(9)
    loads = rng.integers(0, 100, size=(3, E)).astype(np.int32)
    loads[:, 5] = 10**6
    loads[1, 7] = 5 * 10**5
    refs = [oracle.plan(l, lay_o) for l in loads]
    assert max(int(r.logcnt.max()) for r in refs) == 64
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    out = ep.ep_plan_quota(torch.from_numpy(loads).to(dev), lay)
    torch.cuda.synchronize()
    _assert_plan_equal(out, refs)


# The hand-traced run that reaches the move cap (2*S + R = 9 moves), pinned on
# the CPU in tests/test_oracle_plan.py: rank 1 takes replicas of experts 0 and 2
# in its spare slots 3 and 4 (lowest free slot first), and the flag is set.  The
# first layout (one native per rank) runs the rank-per-lane planner; the second
# adds eight idle natives to rank 2, more than the lane planner's eight per rank,
# so the generic LDS planner runs the same moves.
_CAP_CASES = {
    "lanes": (3, [1, 1, 1], list(range(3)), [1, 2, 0], [37, 6, 34]),
    "generic": (11, [1, 1, 9], list(range(11)), [1, 2, 0], [37, 6, 34] + [0] * 8),
}


@pytest.mark.parametrize("kernel", sorted(_CAP_CASES))
def test_plan_step_cap_binds(dev, kernel):
    E, nc, ne, sc, hot = _CAP_CASES[kernel]
    assert (max(nc) > 8) == (kernel == "generic")
    lay_o = oracle.Layout.of(E, 3, nc, ne, sc)
    # plan 0: the cap case; plan 1: the same loads halved (checked against the
    # oracle, whatever it does); plan 2: no load at all
    loads = np.array([hot, [v // 2 for v in hot], [0] * E], np.int32)
    refs = [oracle.plan(l, lay_o) for l in loads]
    assert (refs[0].steps, refs[0].cap_hit) == (9, 1)
    assert refs[0].phy2log.tolist()[:6] == [0, -1, 1, 0, 2, 2]
    assert refs[0].phy_quota.tolist()[:6] == [25, 0, 6, 12, 8, 26]
    print(f"[plan cap] {kernel} E={E}", flush=True)
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    status = torch.full((3,), 0x40, dtype=torch.int32, device=dev)
    out = ep.ep_plan_quota(torch.from_numpy(loads).to(dev), lay, status=status)
    torch.cuda.synchronize()
    _assert_plan_equal(out, refs)
    st = _np(status)
    for p, r in enumerate(refs):
        # the planner ORs its flag into the caller's word and leaves other bits
        assert int(st[p]) == 0x40 | (ep.EP_STATUS_STEP_CAP if r.cap_hit else 0)


@pytest.mark.parametrize("kernel", sorted(_CAP_CASES))
def test_plan_loads_outside_int32(dev, kernel):
    # plans whose loads hold a negative value or sum past INT32_MAX make no
    # move and are flagged; a plan whose total is exactly INT32_MAX is planned
    E, nc, ne, sc, hot = _CAP_CASES[kernel]
    lay_o = oracle.Layout.of(E, 3, nc, ne, sc)
    rows = [hot, [37, -1, 34], [2**31 - 1, 1, 0], [2**30, 2**30, 0], [2**31 - 1 - 10, 10, 0]]
    loads = np.zeros((len(rows), E), np.int64)
    for i, r in enumerate(rows):
        loads[i, :len(r)] = r
    loads = loads.astype(np.int32)
    refs = [oracle.plan(l, lay_o) for l in loads]
    assert [r.bad_load for r in refs] == [0, 1, 1, 1, 0]
    print(f"[plan bad loads] {kernel} E={E}", flush=True)
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    status = torch.zeros((len(rows),), dtype=torch.int32, device=dev)
    out = ep.ep_plan_quota(torch.from_numpy(loads).to(dev), lay, status=status)
    torch.cuda.synchronize()
    _assert_plan_equal(out, refs)
    st = _np(status)
    for p, r in enumerate(refs):
        want = (ep.EP_STATUS_STEP_CAP if r.cap_hit else 0) | (ep.EP_STATUS_BAD_LOAD if r.bad_load else 0)
        assert int(st[p]) == want, p


# --------------------------------------------------------------------- A3
@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_reroute_with_oracle_plan(dev, name):
    wl, wls = _small(name, tokens=45, layers=2, mbs=2)
    lay_o = oracle.Layout.from_workload(wl)
    ids = W.make_ids(wls)
    print(f"[reroute] {name} P={ids.shape[0]} N={ids.shape[1]}", flush=True)
    refs = [oracle.plan(oracle.histogram(ids[p].numpy(), wl.num_experts)[0], lay_o)
            for p in range(ids.shape[0])]
    p2l, q, lc, l2p, _ = _stack_plans(refs)
    lay = ep.Layout.from_workload(wl, device=dev)
    d_ids = ids.to(dev)
    _, ws, _ = ep.ep_load_histogram(d_ids, lay)
    phys = ep.ep_reroute(d_ids, lay, torch.from_numpy(q).to(dev), torch.from_numpy(l2p).to(dev),
                         torch.from_numpy(lc).to(dev), ws)
    torch.cuda.synchronize()
    for p in range(ids.shape[0]):
        ref, unplaced = oracle.reroute(ids[p].numpy(), wl.num_experts, q[p], l2p[p], lc[p])
        assert unplaced == 0
        np.testing.assert_array_equal(_np(phys[p]), ref)


@pytest.mark.parametrize("N", [1, 5, 64, 2047, 2049, 9001, 33000])
def test_reroute_padding_bad_and_short_quota(dev, N):
    rng = np.random.default_rng(77 + N)
    E, R = 21, 5
    nc, ne, sc = [5, 4, 4, 4, 4], list(rng.permutation(E)), [2, 1, 0, 3, 1]
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    P = 2
    ids = torch.from_numpy(rng.choice(E, size=(P, N), p=rng.dirichlet(np.full(E, 0.2))).astype(np.int32))
    ids = W.inject_invalid(ids, E, 0.05, 0.02, seed=N)
    refs = [oracle.plan(oracle.histogram(ids[p].numpy(), E)[0], lay_o) for p in range(P)]
    p2l, q, lc, l2p, _ = _stack_plans(refs)
    q = q.copy()
    # plan 1: shave one unit off a loaded instance so some pairs find no slot
    nz = np.nonzero(q[1] > 0)[0]
    if nz.size:
        q[1, nz[0]] -= 1
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    d_ids = ids.to(dev)
    _, ws, _ = ep.ep_load_histogram(d_ids, lay)
    phys = ep.ep_reroute(d_ids, lay, torch.from_numpy(q).to(dev), torch.from_numpy(l2p).to(dev),
                         torch.from_numpy(lc).to(dev), ws)
    torch.cuda.synchronize()
    for p in range(P):
        ref, _ = oracle.reroute(ids[p].numpy(), E, q[p], l2p[p], lc[p])
        np.testing.assert_array_equal(_np(phys[p]), ref)


def test_reroute_unaligned_rows(dev):
    # N % 4 != 0: rows of later plans are not 16-byte aligned (scalar load path)
    wl = W.get("qwen3_235b")
    E = wl.num_experts
    rng = np.random.default_rng(4)
    N, P = 12345, 3
    ids = torch.from_numpy(rng.integers(0, E, size=(P, N)).astype(np.int32))
    lay_o = oracle.Layout.from_workload(wl)
    lay = ep.Layout.from_workload(wl, device=dev)
    d = ids.to(dev)
    out = ep.run_path(d, lay)
    torch.cuda.synchronize()
    for p in range(P):
        ld, _ = oracle.histogram(ids[p].numpy(), E)
        pl = oracle.plan(ld, lay_o)
        ph, _ = oracle.reroute(ids[p].numpy(), E, pl.phy_quota, pl.log2phy, pl.logcnt)
        np.testing.assert_array_equal(_np(out["load"][p]), ld)
        np.testing.assert_array_equal(_np(out["phys"][p]), ph)


# --------------------------------------------------------------------- A4
@pytest.mark.parametrize("name", ["tiny", "qwen3_235b", "deepseek_v3"])
def test_slot_fill_with_oracle_plan(dev, name):
    wl, wls = _small(name, tokens=64, layers=2)
    lay_o = oracle.Layout.from_workload(wl)
    ids = W.make_ids(wls).numpy()
    elems = 64 * 32 if name == "tiny" else 4096 + 8      # small rows keep the host copy cheap
    w = W.make_weights(wl, device=dev, elems_per_expert=elems)
    w16 = _np(w.view(torch.int16))
    lay = ep.Layout.from_workload(wl, device=dev)
    for p in range(ids.shape[0]):
        pl = oracle.plan(oracle.histogram(ids[p], wl.num_experts)[0], lay_o)
        buf = torch.full((lay.num_spare, elems), 0x7FC1, dtype=torch.int16, device=dev).view(torch.bfloat16)
        ep.ep_slot_fill(w, torch.from_numpy(pl.phy2log).to(dev), lay, buf)
        torch.cuda.synchronize()
        ref = np.full((lay_o.num_spare, elems), 0x7FC1, np.int16)
        oracle.slot_fill(w16, pl.phy2log, lay_o, ref)
        np.testing.assert_array_equal(_np(buf.view(torch.int16)), ref)


@pytest.mark.parametrize("use_ws", [True, False])
@pytest.mark.parametrize("S", [8, 300, 1024, 1025])
def test_slot_fill_replicated_experts(dev, S, use_ws):
    # a few experts fill most spare slots (each read once for all its slots
    # up to 1024 spare slots, slot by slot above), some slots empty; rows of
    # two whole 16 KiB chunks and a tail; with the fill-list workspace and
    # without it
    E, R = 16, 16
    nc, ne = [1] * R, list(range(E))
    sc = [S // R + (1 if r < S % R else 0) for r in range(R)]
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    first, home, rank, spare = lay_o.slots()
    rng = np.random.default_rng(S)
    phy2log = home.astype(np.int32).copy()
    phy2log[spare] = rng.choice([-1, 0, 1, 2, 3, 15], size=S, p=[0.2, 0.3, 0.2, 0.1, 0.1, 0.1])
    elems = 2 * 8192 + 40                               # bf16: 2 chunks of 16 KiB + 80 bytes
    w = rng.integers(0, 1 << 16, size=(E, elems), dtype=np.uint16)
    ref = np.full((S, elems), 0x7FC1, np.uint16)
    oracle.slot_fill(w, phy2log, lay_o, ref)
    buf = torch.from_numpy(np.full((S, elems), 0x7FC1, np.uint16).view(np.int16)).to(dev)
    ep.ep_slot_fill(torch.from_numpy(w.view(np.int16)).to(dev), torch.from_numpy(phy2log).to(dev), lay, buf,
                    use_ws=use_ws)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy().view(np.uint16), ref)


@pytest.mark.parametrize("case", ["one_slot", "one_expert_everywhere", "all_empty", "one_vector",
                                  "ws_reused"])
def test_slot_fill_list_edges(dev, case):
    # the fill list at its edges: a single spare slot, one expert in every
    # slot (64 stores per chunk), no expert at all, 16-byte experts (one
    # vector, one partial workgroup), and one workspace reused by plans with
    # fewer and more distinct experts than the last
    E, R = 64, 64
    nc, ne = [1] * R, list(range(E))
    sc = [1 if (case != "one_slot" or r == 5) else 0 for r in range(R)]
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    first, home, rank, spare = lay_o.slots()
    S = len(spare)
    rng = np.random.default_rng(21)
    elems = 8 if case == "one_vector" else 2048 * 3 + 8
    w = rng.integers(0, 1 << 16, size=(E, elems), dtype=np.uint16)
    d_w = torch.from_numpy(w.view(np.int16)).to(dev)
    ws = ep.slot_fill_workspace(lay, dev)
    ws.fill_(0x55)
    plans = []
    if case == "one_expert_everywhere":
        plans.append(np.full(S, 7))
    elif case == "all_empty":
        plans.append(np.full(S, -1))
    elif case == "ws_reused":
        plans += [rng.integers(-1, 4, size=S), rng.integers(-1, E, size=S), np.full(S, 3), rng.integers(-1, 2, size=S)]
    else:
        plans.append(rng.integers(0, E, size=S))
    for sp in plans:
        phy2log = home.astype(np.int32).copy()
        phy2log[spare] = sp
        ref = np.full((S, elems), 0x7FC1, np.uint16)
        oracle.slot_fill(w, phy2log, lay_o, ref)
        buf = torch.from_numpy(np.full((S, elems), 0x7FC1, np.uint16).view(np.int16)).to(dev)
        ep.ep_slot_fill(d_w, torch.from_numpy(phy2log).to(dev), lay, buf, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(buf.cpu().numpy().view(np.uint16), ref)


@pytest.mark.parametrize("use_ws", [True, False])
@pytest.mark.parametrize("S", [8, 1025])
def test_slot_fill_entries_naming_no_expert(dev, S, use_ws):
    # spare entries outside [0, E) (E, E + 7, INT32_MAX) name no expert: their
    # rows keep the sentinel, in the shared fill (S <= 1024) and the per-slot one
    E, R = 16, 16
    nc, ne = [1] * R, list(range(E))
    sc = [S // R + (1 if r < S % R else 0) for r in range(R)]
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    first, home, rank, spare = lay_o.slots()
    rng = np.random.default_rng(100 + S)
    phy2log = home.astype(np.int32).copy()
    phy2log[spare] = rng.choice([-1, 0, 5, 15, E, E + 7, 2 ** 31 - 1], size=S)
    elems = 8192 + 24
    w = rng.integers(0, 1 << 16, size=(E, elems), dtype=np.uint16)
    ref = np.full((S, elems), 0x7FC1, np.uint16)
    oracle.slot_fill(w, phy2log, lay_o, ref)
    buf = torch.from_numpy(np.full((S, elems), 0x7FC1, np.uint16).view(np.int16)).to(dev)
    ep.ep_slot_fill(torch.from_numpy(w.view(np.int16)).to(dev), torch.from_numpy(phy2log).to(dev), lay, buf,
                    use_ws=use_ws)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy().view(np.uint16), ref)


# --------------------------------------------------------------------- A5
@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_stats_with_oracle_inputs(dev, name):
    wl, wls = _small(name, tokens=50, layers=3)
    lay_o = oracle.Layout.from_workload(wl)
    ids = W.make_ids(wls).numpy()
    loads = np.stack([oracle.histogram(ids[p], wl.num_experts)[0] for p in range(ids.shape[0])])
    plans = [oracle.plan(l, lay_o) for l in loads]
    quotas = np.stack([p.phy_quota for p in plans])
    lay = ep.Layout.from_workload(wl, device=dev)
    st, imb, rl = ep.ep_balance_stats(torch.from_numpy(loads).to(dev), torch.from_numpy(quotas).to(dev), lay)
    torch.cuda.synchronize()
    for p in range(loads.shape[0]):
        ref = oracle.stats(loads[p], quotas[p], lay_o)
        np.testing.assert_array_equal(_np(st[p]), ref.as_row())
        assert _np(imb[p]).tolist() == [ref.imbalance_before, ref.imbalance_after]
        np.testing.assert_array_equal(_np(rl[p, 0]), ref.rank_before)
        np.testing.assert_array_equal(_np(rl[p, 1]), ref.rank_after)


def test_stats_zero_load(dev):
    wl = W.get("tiny")
    lay = ep.Layout.from_workload(wl, device=dev)
    z = torch.zeros((1, 12), dtype=torch.int32, device=dev)
    q = torch.zeros((1, 16), dtype=torch.int32, device=dev)
    st, imb, _ = ep.ep_balance_stats(z, q, lay)
    torch.cuda.synchronize()
    assert _np(st[0]).tolist() == [0, 0, 0, 0] and _np(imb[0]).tolist() == [1.0, 1.0]


# --------------------------------------------------------------------- chain
@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_full_chain_small(dev, name):
    wl, wls = _small(name, tokens=41, layers=3, mbs=2)
    lay_o = oracle.Layout.from_workload(wl)
    ids = W.make_ids(wls)
    lay = ep.Layout.from_workload(wl, device=dev)
    out = ep.run_path(ids.to(dev), lay)
    torch.cuda.synchronize()
    ref = oracle.run_path(ids.numpy(), lay_o)
    np.testing.assert_array_equal(_np(out["load"]), ref["load"])
    _assert_plan_equal(out["plan"], ref["plans"])
    np.testing.assert_array_equal(_np(out["phys"]), ref["phys"])
    np.testing.assert_array_equal(_np(out["stats"]), np.stack([s.as_row() for s in ref["stats"]]))


def test_empty_and_all_padding(dev):
    wl = W.get("tiny")
    lay = ep.Layout.from_workload(wl, device=dev)
    lay_o = oracle.Layout.from_workload(wl)
    for N in (0, 300):
        ids = torch.full((2, N), -1, dtype=torch.int32)
        out = ep.run_path(ids.to(dev), lay)
        torch.cuda.synchronize()
        assert int(out["load"].abs().sum()) == 0
        ref = oracle.plan(np.zeros(12, np.int32), lay_o)
        _assert_plan_equal(out["plan"], [ref, ref])
        if N:
            assert bool((out["phys"] == -1).all())


def test_deterministic_and_stream_independent(dev):
    wl, wls = _small("stress", tokens=300, layers=2, mbs=1)
    lay = ep.Layout.from_workload(wl, device=dev)
    ids = W.make_ids(wls, device=dev)
    a = ep.run_path(ids, lay)
    s2 = torch.cuda.Stream()
    # the IDs come from work on the current stream: the side stream waits for it
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s2):
        b = ep.run_path(ids, lay)
    s2.synchronize()
    torch.cuda.synchronize()
    for k in ("load", "phys", "stats"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["plan"].log2phy, b["plan"].log2phy)
    assert torch.equal(a["plan"].phy_quota, b["plan"].phy_quota)


# ------------------------------------------------ planner kernel selection
# The library plans with one rank per lane when R <= 64, every rank has at
# most 8 natives (1, 2, 4, 6 or 8 native registers per lane) and at most 16
# spare slots (1, 2, 4, 8 or 16 spare registers), and with the generic LDS
# kernel otherwise; both must agree with the oracle.  The rank-per-lane
# kernel picks candidates with scalar compares when natives + spares per lane
# <= 5 ((4, 1), (1, 4), (2, 2), (1, 1) below) and with wave reductions above.
@pytest.mark.parametrize("R,E,max_sp", [(8, 20, 1), (16, 40, 2), (24, 50, 3), (32, 64, 7),
                                        (12, 30, 13), (70, 140, 1), (90, 90, 0), (4, 12, 20),
                                        (16, 80, 3), (10, 55, 2), (8, 60, 1), (6, 54, 2),
                                        (16, 16, 4), (32, 64, 2), (64, 64, 1)])
def test_plan_kernel_paths(dev, R, E, max_sp):
    rng = np.random.default_rng(R * 1000 + E)
    nc = np.full(R, E // R)
    nc[: E % R] += 1
    ne = rng.permutation(E)
    sc = rng.integers(0, max_sp + 1, size=R)
    sc[0] = max_sp
    S = int(sc.sum())
    if min(R, 1 + S) > 64:                      # keep rho within the planner's limit
        sc[:] = 0
        sc[: 63] = 1
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    P = 5
    loads = (rng.pareto(0.7, size=(P, E)) * 100).astype(np.int32)
    loads[0] = 0
    loads[1, rng.integers(0, E)] = 10**6
    refs = [oracle.plan(l, lay_o) for l in loads]
    print(f"[plan-path] R={R} E={E} max_spare={int(sc.max())} steps={[r.steps for r in refs]}", flush=True)
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    status = torch.zeros(P, dtype=torch.int32, device=dev)
    out = ep.ep_plan_quota(torch.from_numpy(loads).to(dev), lay, status=status)
    torch.cuda.synchronize()
    _assert_plan_equal(out, refs)
    np.testing.assert_array_equal(_np(status), [ep.EP_STATUS_STEP_CAP if r.cap_hit else 0 for r in refs])


def test_reroute_many_split_experts_in_one_subblock(dev):
    # 200 experts on 64 ranks with 3 spare slots each, and a plan built by hand:
    # experts 0..119 get a replica in a spare slot of another rank and half of
    # their 16 pairs each; the other 80 experts carry 1 pair.  The plan's 2000
    # pairs fit one sub-block (2048 pairs at E = 200 and one plan), in which
    # 120 experts have a quota boundary (the reroute keeps 64 of them in
    # registers and the rest in LDS).
    E, R, S = 200, 64, 3
    nc = [4] * 8 + [3] * 56
    first = np.concatenate([[0], np.cumsum([n + S for n in nc])])
    Phi = int(first[-1])
    rho = min(R, 1 + S * R)
    native = np.concatenate([first[r] + np.arange(nc[r]) for r in range(R)])  # expert e's native slot
    rank_of = np.repeat(np.arange(R), nc)
    cnt = np.where(np.arange(E) < 120, 16, 1)
    q = np.zeros(Phi, np.int32)
    l2p = np.full((E, rho), -1, np.int32)
    lc = np.ones(E, np.int32)
    used = np.zeros(R, np.int64)
    for e in range(E):
        if e < 120:
            r = (rank_of[e] + 1 + e % 7) % R          # another rank with a free spare slot
            while used[r] >= S or r == rank_of[e]:
                r = (r + 1) % R
            rs = first[r] + nc[r] + used[r]
            used[r] += 1
            a, b = sorted([native[e], rs])
            l2p[e, :2] = [a, b]
            lc[e] = 2
            q[a], q[b] = 8, 8
        else:
            l2p[e, 0] = native[e]
            q[native[e]] = cnt[e]
    rng = np.random.default_rng(21)
    ids = rng.permutation(np.repeat(np.arange(E), cnt)).astype(np.int32)[None]
    assert ids.shape[1] <= 2048
    lay = ep.Layout.create(E, nc, list(range(E)), [S] * R, device=dev)
    assert lay.num_phys == Phi and lay.max_replicas == rho
    d_ids = torch.from_numpy(ids).to(dev)
    _, ws, _ = ep.ep_load_histogram(d_ids, lay)
    phys = ep.ep_reroute(d_ids, lay, torch.from_numpy(q[None]).to(dev), torch.from_numpy(l2p[None]).to(dev),
                         torch.from_numpy(lc[None]).to(dev), ws)
    torch.cuda.synchronize()
    ref, unplaced = oracle.reroute(ids[0], E, q, l2p, lc)
    assert unplaced == 0
    np.testing.assert_array_equal(_np(phys[0]), ref)


# ------------------------------------------------ domain-constrained planner
@pytest.mark.parametrize("name,D", [("qwen3_235b", 8), ("deepseek_v3", 8), ("glm_4_5", 8), ("stress", 8),
                                    ("tiny", 2), ("qwen3_235b", 1), ("stress", 64)])
def test_plan_domain_matches_oracle(dev, name, D):
    wl, wls = _small(name, tokens=200, layers=3, mbs=2)
    lay_o = oracle.Layout.from_workload(wl)
    ids = W.make_ids(wls).numpy()
    loads = np.stack([oracle.histogram(ids[p], wl.num_experts)[0] for p in range(ids.shape[0])])
    refs = [oracle.plan(l, lay_o, D) for l in loads]
    lay = ep.Layout.from_workload(wl, device=dev).with_domain(D)
    out = ep.ep_plan_quota(torch.from_numpy(loads).to(dev), lay)
    torch.cuda.synchronize()
    _assert_plan_equal(out, refs)


@pytest.mark.parametrize("seed", range(3))
def test_plan_domain_random_layouts(dev, seed):
    # random layouts hit both planner kernels (rank-per-lane and generic)
    rng = np.random.default_rng(500 + seed)
    for it in range(8):
        E, R, nc, ne, sc = W.random_layout(rng, max_experts=90, max_ranks=80, max_spare_per_rank=3)
        lay_o = oracle.Layout.of(E, R, nc, ne, sc)
        if lay_o.max_replicas > 64:
            continue
        D = int(rng.integers(1, R + 1))
        loads = (rng.pareto(0.8, size=(2, E)) * 60).astype(np.int32)
        refs = [oracle.plan(l, lay_o, D) for l in loads]
        lay = ep.Layout.create(E, nc, ne, sc, device=dev).with_domain(D)
        out = ep.ep_plan_quota(torch.from_numpy(loads).to(dev), lay)
        torch.cuda.synchronize()
        _assert_plan_equal(out, refs)


def test_binding_rejects_wrong_shapes(dev):
    # the kernels trust the sizes, so the binding checks every tensor's shape
    wl = W.get("tiny")
    lay = ep.Layout.from_workload(wl, device=dev)
    ids = W.make_ids(wl).to(dev)
    P, N = ids.shape
    E, Phi, rho = lay.num_experts, lay.num_phys, lay.max_replicas
    load, ws, status = ep.ep_load_histogram(ids, lay)
    with pytest.raises(ep.EPBalanceError):
        ep.ep_load_histogram(ids, lay, load=torch.empty((P, E - 1), dtype=torch.int32, device=dev))
    with pytest.raises(ep.EPBalanceError):
        ep.ep_load_histogram(ids, lay, ws=ws[:4])
    bad = ep.alloc_plan(P, lay, dev)
    bad.log2phy = torch.empty((P, E, rho - 1), dtype=torch.int32, device=dev)
    with pytest.raises(ep.EPBalanceError):
        ep.ep_plan_quota(load, lay, out=bad)
    plan = ep.ep_plan_quota(load, lay)
    with pytest.raises(ep.EPBalanceError):
        ep.ep_reroute(ids, lay, plan.phy_quota[:, :-1].contiguous(), plan.log2phy, plan.logcnt, ws)
    with pytest.raises(ep.EPBalanceError):
        ep.ep_reroute(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws,
                      phys_ids=torch.empty((P, N - 1), dtype=torch.int32, device=dev))
    with pytest.raises(ep.EPBalanceError):
        ep.ep_dispatch_layout(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws,
                              slot_offsets=torch.empty((P, Phi), dtype=torch.int32, device=dev))
    with pytest.raises(ep.EPBalanceError):
        ep.ep_balance_stats(load, plan.phy_quota, lay, stats=torch.empty((P, 4), dtype=torch.int32, device=dev))
    with pytest.raises(ep.EPBalanceError):
        ep.ep_slot_fill(torch.empty((E, 64), dtype=torch.bfloat16, device=dev), plan.phy2log[0][:-1].contiguous(),
                        lay, torch.empty((lay.num_spare, 64), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ep.EPBalanceError):
        ep.ep_replica_grad_reduce(torch.zeros((E, 8), device=dev), torch.zeros((lay.num_spare, 4), device=dev),
                                  plan.log2phy[0].contiguous(), plan.logcnt[0].contiguous(), lay)
    # the shapes the path itself uses still pass
    ep.ep_reroute(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws)
    torch.cuda.synchronize()
