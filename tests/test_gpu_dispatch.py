"""GPU parity of the dispatch layout (slot-major pair order, inverse positions,
slot offsets) against the CPU oracle, bit-exact."""
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


def _np(t):
    return t.detach().cpu().numpy()


def _check(ids_h, E, plans, off, pos, src):
    for p, pl in enumerate(plans):
        ro, rp, rs, _ = oracle.dispatch(ids_h[p], E, pl.phy_quota, pl.log2phy, pl.logcnt)
        np.testing.assert_array_equal(_np(off[p]).astype(np.int64), ro)
        np.testing.assert_array_equal(_np(pos[p]), rp)
        np.testing.assert_array_equal(_np(src[p]), rs)


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_dispatch_with_oracle_plan(dev, name):
    wl = W.get(name)
    wls = wl.scaled(tokens_per_rank=min(wl.tokens_per_rank, 45), layers=min(wl.layers, 2),
                    microbatches=min(wl.microbatches, 2))
    lay_o = oracle.Layout.from_workload(wl)
    ids = W.inject_invalid(W.make_ids(wls), wl.num_experts, 0.02, 0.01)
    ids_h = ids.numpy()
    print(f"[dispatch] {name} P={ids.shape[0]} N={ids.shape[1]}", flush=True)
    plans = [oracle.plan(oracle.histogram(ids_h[p], wl.num_experts)[0], lay_o) for p in range(ids.shape[0])]
    lay = ep.Layout.from_workload(wl, device=dev)
    d = ids.to(dev)
    _, ws, _ = ep.ep_load_histogram(d, lay)
    st = lambda k: torch.from_numpy(np.stack([getattr(pl, k) for pl in plans])).to(dev)
    off, pos, src = ep.ep_dispatch_layout(d, lay, st("phy_quota"), st("log2phy"), st("logcnt"), ws)
    torch.cuda.synchronize()
    _check(ids_h, wl.num_experts, plans, off, pos, src)


@pytest.mark.parametrize("N", [0, 1, 63, 2049, 12345])
def test_dispatch_edges(dev, N):
    rng = np.random.default_rng(31 + N)
    E, R = 21, 5
    nc, ne, sc = [5, 4, 4, 4, 4], list(rng.permutation(E)), [2, 1, 0, 3, 1]
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    P = 2
    ids = torch.from_numpy(rng.choice(E, size=(P, N), p=rng.dirichlet(np.full(E, 0.2))).astype(np.int32))
    if N:
        ids = W.inject_invalid(ids, E, 0.05, 0.02, seed=N)
    ids_h = ids.numpy()
    plans = [oracle.plan(oracle.histogram(ids_h[p], E)[0], lay_o) for p in range(P)]
    if N > 10:
        # plan 1: one instance gets one unit less, so one pair finds no slot
        q = plans[1].phy_quota
        nz = np.nonzero(q > 0)[0]
        q[nz[-1]] -= 1
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    d = ids.to(dev)
    _, ws, _ = ep.ep_load_histogram(d, lay)
    st = lambda k: torch.from_numpy(np.stack([getattr(pl, k) for pl in plans])).to(dev)
    off, pos, src = ep.ep_dispatch_layout(d, lay, st("phy_quota"), st("log2phy"), st("logcnt"), ws)
    torch.cuda.synchronize()
    _check(ids_h, E, plans, off, pos, src)


@pytest.mark.parametrize("N", [40, 5000])
def test_dispatch_over_quota_plan(dev, N):
    # quotas above the loads: an instance in the middle of an expert's list and
    # the last instance of another get extra units, so positions inside the
    # layout (not only past its end) are taken by no pair and must hold -1
    rng = np.random.default_rng(77 + N)
    E, R = 10, 4
    nc, ne, sc = [3, 3, 2, 2], list(range(E)), [2, 2, 1, 1]
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    ids = torch.from_numpy(rng.choice(3, size=(1, N), p=[0.6, 0.3, 0.1]).astype(np.int32))
    ids_h = ids.numpy()
    pl = oracle.plan(oracle.histogram(ids_h[0], E)[0], lay_o)
    multi = [e for e in range(E) if pl.logcnt[e] >= 2]
    assert multi, "the skewed load should replicate an expert"
    e0 = multi[0]
    pl.phy_quota[pl.log2phy[e0, 0]] += 5          # a gap before e0's second instance
    pl.phy_quota[pl.log2phy[1, pl.logcnt[1] - 1]] += 3
    ro, rp, rs, placed = oracle.dispatch(ids_h[0], E, pl.phy_quota, pl.log2phy, pl.logcnt)
    assert placed == N and np.any((rs[:-1] == -1) & (rs[1:] >= 0))   # a gap inside the layout
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    d = ids.to(dev)
    _, ws, _ = ep.ep_load_histogram(d, lay)
    st = lambda k: torch.from_numpy(getattr(pl, k)[None].copy()).to(dev)
    src_junk = torch.full((1, N), 12345, dtype=torch.int32, device=dev)
    off, pos, src = ep.ep_dispatch_layout(d, lay, st("phy_quota"), st("log2phy"), st("logcnt"), ws,
                                          dispatch_src=src_junk)
    torch.cuda.synchronize()
    _check(ids_h, E, [pl], off, pos, src)


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_dispatch_fullsize_chain(dev, name):
    wl = W.get(name)
    print(f"[dispatch-fullsize] {name}: P={wl.num_plans} N={wl.pairs_per_plan}", flush=True)
    ids = W.make_ids(wl, device=dev)
    lay = ep.Layout.from_workload(wl, device=dev)
    out = ep.run_path(ids, lay)
    pl = out["plan"]
    off, pos, src = ep.ep_dispatch_layout(ids, lay, pl.phy_quota, pl.log2phy, pl.logcnt, out["ws"])
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    del ids, out
    torch.cuda.empty_cache()
    lay_o = oracle.Layout.from_workload(wl)
    plans = [oracle.plan(oracle.histogram(ids_h[p], wl.num_experts)[0], lay_o) for p in range(wl.num_plans)]
    _check(ids_h, wl.num_experts, plans, off, pos, src)
