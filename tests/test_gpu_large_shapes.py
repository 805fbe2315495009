"""Layouts at the edges of what the kernels hold in LDS: many experts, many
ranks (the generic planner), and the largest histogram.  Each runs the chain
on the GPU and compares it with the CPU oracle bit for bit; shapes beyond a
kernel's limit must be rejected, not run."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

ep = pytest.importorskip("moe_expert_load_layer_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _layout(E, R, S, seed):
    rng = np.random.default_rng(seed)
    nc = np.full(R, E // R)
    nc[: E % R] += 1
    ne = rng.permutation(E)
    sc = np.zeros(R, np.int64)
    sc[rng.permutation(R)[:S]] = 1
    return [int(x) for x in nc], [int(x) for x in ne], [int(x) for x in sc]


def _ids(E, P, N, seed):
    rng = np.random.default_rng(seed)
    out = np.empty((P, N), np.int32)
    for p in range(P):
        cdf = np.cumsum(rng.dirichlet(np.full(E, 0.2)))
        out[p] = np.minimum(np.searchsorted(cdf, rng.random(N), side="right"), E - 1)
    out[:, ::211] = -1
    return out


@pytest.mark.parametrize("E,R,S", [(1500, 100, 63), (1024, 1024, 63), (1200, 64, 63), (2048, 2048, 63),
                                   (3000, 200, 63)])
def test_large_layouts_full_chain(dev, E, R, S):
    # (1500, 100) and (1024, 1024): the generic planner with a 64 KiB table;
    # (1200, 64): 19 natives per rank, also the generic planner; (2048, 2048)
    # and (3000, 200): tables of 122 KiB and 123 KiB, beyond 64 KiB of LDS
    # (gfx950 gives a workgroup up to 160 KiB), with the reroute and the
    # dispatch layout at 2048 and 3000 experts
    nc, ne, sc = _layout(E, R, S, E + R)
    P, N = 2, 300_007
    ids_h = _ids(E, P, N, E * 7 + R)
    print(f"[large] E={E} R={R} S={S} P={P} N={N}", flush=True)
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    ids = torch.from_numpy(ids_h).to(dev)
    out = ep.run_path(ids, lay)
    pl = out["plan"]
    off, pos, src = ep.ep_dispatch_layout(ids, lay, pl.phy_quota, pl.log2phy, pl.logcnt, out["ws"])
    torch.cuda.synchronize()
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    for p in range(P):
        ld, _ = oracle.histogram(ids_h[p], E)
        assert np.array_equal(out["load"][p].cpu().numpy(), ld)
        r = oracle.plan(ld, lay_o)
        assert np.array_equal(pl.phy_quota[p].cpu().numpy(), r.phy_quota)
        assert np.array_equal(pl.log2phy[p].cpu().numpy(), r.log2phy)
        assert int(pl.steps[p]) == r.steps
        ph, _ = oracle.reroute(ids_h[p], E, r.phy_quota, r.log2phy, r.logcnt)
        assert np.array_equal(out["phys"][p].cpu().numpy(), ph)
        ro, rp, rs, _ = oracle.dispatch(ids_h[p], E, r.phy_quota, r.log2phy, r.logcnt)
        assert np.array_equal(off[p].cpu().numpy().astype(np.int64), ro)
        assert np.array_equal(pos[p].cpu().numpy(), rp)
        assert np.array_equal(src[p].cpu().numpy(), rs)


def test_largest_histogram_and_reroute(dev):
    # E = 5119 fills the histogram's 160 KiB of LDS exactly (8 waves x 5120
    # counters); 80 natives per rank are beyond both planner kernels (the
    # generic planner's tables would take 203 KiB), so the planner must
    # refuse and the reroute runs on the oracle's plan
    E, R, S = 5119, 64, 64
    nc, ne, sc = _layout(E, R, S, 9)
    P, N = 2, 400_003
    ids_h = _ids(E, P, N, 11)
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    ids = torch.from_numpy(ids_h).to(dev)
    load, ws, status = ep.ep_load_histogram(ids, lay)
    with pytest.raises(ep.EPBalanceError):
        ep.ep_plan_quota(load, lay)
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    plans = [oracle.plan(oracle.histogram(ids_h[p], E)[0], lay_o) for p in range(P)]
    st = lambda k: torch.from_numpy(np.stack([getattr(r, k) for r in plans])).to(dev)
    phys = ep.ep_reroute(ids, lay, st("phy_quota"), st("log2phy"), st("logcnt"), ws)
    torch.cuda.synchronize()
    for p in range(P):
        ld, _ = oracle.histogram(ids_h[p], E)
        assert np.array_equal(load[p].cpu().numpy(), ld)
        ph, _ = oracle.reroute(ids_h[p], E, plans[p].phy_quota, plans[p].log2phy, plans[p].logcnt)
        assert np.array_equal(phys[p].cpu().numpy(), ph)
    # one expert more is beyond the histogram's LDS
    nc2, ne2, sc2 = _layout(E + 1, R, S, 10)
    lay2 = ep.Layout.create(E + 1, nc2, ne2, sc2, device=dev)
    with pytest.raises(ep.EPBalanceError):
        ep.ep_load_histogram(ids, lay2)


def test_most_plans_per_call(dev):
    # P = 65535 plans (the grid's y extent) of 13 pairs each on the Tiny layout
    E, R = 12, 8
    nc, ne, sc = [2, 2, 2, 2, 1, 1, 1, 1], list(range(12)), [0, 0, 0, 0, 1, 1, 1, 1]
    P, N = 65535, 13
    rng = np.random.default_rng(65535)
    ids_h = rng.integers(-1, E, size=(P, N), dtype=np.int32)
    ids_h[:, 0] = rng.integers(0, 3, size=P)           # a hot expert per plan
    print(f"[plans] P={P} N={N}", flush=True)
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    ids = torch.from_numpy(ids_h).to(dev)
    out = ep.run_path(ids, lay)
    torch.cuda.synchronize()
    load = out["load"].cpu().numpy(); q = out["plan"].phy_quota.cpu().numpy()
    phys = out["phys"].cpu().numpy(); st = out["stats"].cpu().numpy()
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    for p in list(range(0, P, 97)) + [P - 1]:
        ld, _ = oracle.histogram(ids_h[p], E)
        assert np.array_equal(load[p], ld), p
        r = oracle.plan(ld, lay_o)
        assert np.array_equal(q[p], r.phy_quota), p
        ph, _ = oracle.reroute(ids_h[p], E, r.phy_quota, r.log2phy, r.logcnt)
        assert np.array_equal(phys[p], ph), p
        assert np.array_equal(st[p], oracle.stats(ld, r.phy_quota, lay_o).as_row()), p
    # every plan's loads are exact (a property that holds at any size)
    ref = np.stack([np.bincount(row[row >= 0], minlength=E) for row in ids_h])
    assert np.array_equal(load, ref)
    with pytest.raises(ep.EPBalanceError):
        ep.ep_load_histogram(torch.zeros((P + 1, N), dtype=torch.int32, device=dev), lay)


def test_most_spare_slots_in_slot_fill(dev):
    # 65535 spare slots (the slot fill's grid y extent), every one given a
    # random expert or left empty; one slot more is refused
    E, R = 64, 64
    S = 65535
    nc, ne = [1] * R, list(range(E))
    sc = [S // R + (1 if r < S % R else 0) for r in range(R)]
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    first, home, rank, spare = lay_o.slots()
    rng = np.random.default_rng(4)
    phy2log = home.astype(np.int32).copy()
    phy2log[spare] = rng.integers(-1, E, size=S)
    w = rng.integers(0, 1 << 16, size=(E, 48), dtype=np.uint16)
    ref = np.full((S, 48), 0x7FC1, np.uint16)
    oracle.slot_fill(w, phy2log, lay_o, ref)
    buf = torch.from_numpy(np.full((S, 48), 0x7FC1, np.uint16).view(np.int16)).to(dev)
    ep.ep_slot_fill(torch.from_numpy(w.view(np.int16)).to(dev), torch.from_numpy(phy2log).to(dev), lay, buf)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy().view(np.uint16), ref)
    sc2 = list(sc)
    sc2[0] += 1
    lay2 = ep.Layout.create(E, nc, ne, sc2, device=dev)
    with pytest.raises(ep.EPBalanceError):
        ep.ep_slot_fill(torch.from_numpy(w.view(np.int16)).to(dev),
                        torch.zeros(lay2.num_phys, dtype=torch.int32, device=dev), lay2,
                        torch.zeros((S + 1, 48), dtype=torch.int16, device=dev))
