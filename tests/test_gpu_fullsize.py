"""Full-size parity: every workload at its full size, all plans in one launch
(the launch configuration bench.py times), against the CPU oracle.

Histogram, plan, reroute and statistics are compared in full.  The slot fill
(gigabytes per layer) is compared byte for byte on the device: every used spare
slot's row must equal the weights row of the expert the oracle's plan puts
there, and every empty slot's row must keep its sentinel bytes; sampled windows
are also brought to the host and compared there.
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


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_fullsize_path(dev, name):
    wl = W.get(name)
    print(f"[fullsize] {name}: P={wl.num_plans} N={wl.pairs_per_plan}", flush=True)
    ids = W.make_ids(wl, device=dev)
    lay = ep.Layout.from_workload(wl, device=dev)
    out = ep.run_path(ids, lay)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    del ids
    load = out["load"].cpu().numpy()
    phys = out["phys"].cpu().numpy()
    st = out["stats"].cpu().numpy()
    imb = out["imbalance"].cpu().numpy()
    status = out["status"].cpu().numpy()
    plan = {k: getattr(out["plan"], k).cpu().numpy() for k in ("phy2log", "phy_quota", "logcnt", "log2phy", "steps")}
    del out
    torch.cuda.empty_cache()
    lay_o = oracle.Layout.from_workload(wl)
    for p in range(wl.num_plans):
        ld, bad = oracle.histogram(ids_h[p], wl.num_experts)
        assert np.array_equal(load[p], ld), f"load plan {p}"
        pl = oracle.plan(ld, lay_o)
        assert np.array_equal(plan["phy2log"][p], pl.phy2log), f"phy2log plan {p}"
        assert np.array_equal(plan["phy_quota"][p], pl.phy_quota), f"quota plan {p}"
        assert np.array_equal(plan["logcnt"][p], pl.logcnt), f"logcnt plan {p}"
        assert np.array_equal(plan["log2phy"][p], pl.log2phy), f"log2phy plan {p}"
        assert plan["steps"][p] == pl.steps
        assert status[p] == (ep.EP_STATUS_STEP_CAP if pl.cap_hit else 0) | (ep.EP_STATUS_BAD_ID if bad else 0)
        ph, _ = oracle.reroute(ids_h[p], wl.num_experts, pl.phy_quota, pl.log2phy, pl.logcnt)
        assert np.array_equal(phys[p], ph), f"reroute plan {p}"
        s = oracle.stats(ld, pl.phy_quota, lay_o)
        assert np.array_equal(st[p], s.as_row()), f"stats plan {p}"
        assert imb[p].tolist() == [s.imbalance_before, s.imbalance_after]


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_fullsize_single_layer(dev, name):
    # one full-size plan per launch, as a forward pass without batching calls
    # the path: the library then cuts the plan into smaller sub-blocks (2048
    # pairs at E = 128) than in the batched launch; dispatch layout included
    wl = W.get(name)
    E = wl.num_experts
    p0 = wl.num_plans - 1
    ids = W.make_ids(wl, device=dev, plans=[p0])
    print(f"[fullsize-1] {name}: plan {p0}, N={ids.shape[1]}", flush=True)
    lay = ep.Layout.from_workload(wl, device=dev)
    out = ep.run_path(ids, lay)
    pl_g = out["plan"]
    off, pos, src = ep.ep_dispatch_layout(ids, lay, pl_g.phy_quota, pl_g.log2phy, pl_g.logcnt, out["ws"])
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()[0]
    lay_o = oracle.Layout.from_workload(wl)
    ld, bad = oracle.histogram(ids_h, E)
    assert np.array_equal(out["load"][0].cpu().numpy(), ld)
    pl = oracle.plan(ld, lay_o)
    for k in ("phy2log", "phy_quota", "logcnt", "log2phy"):
        assert np.array_equal(getattr(pl_g, k)[0].cpu().numpy(), getattr(pl, k)), k
    assert int(pl_g.steps[0]) == pl.steps
    assert int(out["status"][0]) == (ep.EP_STATUS_STEP_CAP if pl.cap_hit else 0) | (ep.EP_STATUS_BAD_ID if bad else 0)
    ph, _ = oracle.reroute(ids_h, E, pl.phy_quota, pl.log2phy, pl.logcnt)
    assert np.array_equal(out["phys"][0].cpu().numpy(), ph)
    ro, rp, rs, _ = oracle.dispatch(ids_h, E, pl.phy_quota, pl.log2phy, pl.logcnt)
    assert np.array_equal(off[0].cpu().numpy().astype(np.int64), ro)
    assert np.array_equal(pos[0].cpu().numpy(), rp)
    assert np.array_equal(src[0].cpu().numpy(), rs)


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_fullsize_slot_fill(dev, name):
    wl = W.get(name)
    print(f"[fullsize-fill] {name}: E={wl.num_experts} S={wl.num_spare} bytes/expert={wl.bytes_per_expert}",
          flush=True)
    lay = ep.Layout.from_workload(wl, device=dev)
    lay_o = oracle.Layout.from_workload(wl)
    _, _, _, spare = lay_o.slots()
    plans = [0, wl.num_plans - 1]
    ids = W.make_ids(wl, device=dev, plans=plans)
    weights = W.make_weights(wl, device=dev)
    w16 = weights.view(torch.int16)
    slot = torch.empty((wl.num_spare, weights.shape[1]), dtype=weights.dtype, device=dev)
    s16 = slot.view(torch.int16)
    rng = np.random.default_rng(5)
    elems = weights.shape[1]
    win = 2048                                  # int16 elements per window (4 KiB)
    for i, p in enumerate(plans):
        ld, _ = oracle.histogram(ids[i].cpu().numpy(), wl.num_experts)
        pl = oracle.plan(ld, lay_o)
        s16.fill_(0x7FC1)
        ep.ep_slot_fill(weights, torch.from_numpy(pl.phy2log).to(dev), lay, slot)
        torch.cuda.synchronize()
        # every byte, on the device
        for o, s in enumerate(spare):
            e = int(pl.phy2log[s])
            if e >= 0:
                assert torch.equal(s16[o], w16[e]), f"plan {p} slot {o} expert {e}"
            else:
                assert bool((s16[o] == 0x7FC1).all()), f"plan {p} empty slot {o} was written"
        for o, s in enumerate(spare):
            e = int(pl.phy2log[s])
            starts = list(rng.integers(0, max(1, elems - win), size=6) // 8 * 8) + [0, max(0, elems - win)]
            for a in starts:
                got = s16[o, a:a + win].cpu().numpy()
                if e >= 0:
                    exp = w16[e, a:a + win].cpu().numpy()
                    assert np.array_equal(got, exp), f"plan {p} slot {o} expert {e} window {a}"
                else:
                    assert np.all(got == 0x7FC1), f"plan {p} empty slot {o} was written"
    del weights, slot
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["qwen3_235b", "deepseek_v3"])
def test_fullsize_domain_plan(dev, name):
    # all plans in one launch with replicas confined to 8-rank domains
    wl = W.get(name)
    print(f"[fullsize-domain] {name}: P={wl.num_plans} R={wl.num_ranks} D=8", flush=True)
    ids = W.make_ids(wl, device=dev)
    lay = ep.Layout.from_workload(wl, device=dev).with_domain(8)
    load, _, _ = ep.ep_load_histogram(ids, lay)
    out = ep.ep_plan_quota(load, lay)
    torch.cuda.synchronize()
    del ids
    load_h = load.cpu().numpy()
    got = {k: getattr(out, k).cpu().numpy() for k in ("phy2log", "phy_quota", "logcnt", "log2phy", "steps")}
    lay_o = oracle.Layout.from_workload(wl)
    for p in range(wl.num_plans):
        pl = oracle.plan(load_h[p], lay_o, 8)
        for k in ("phy2log", "phy_quota", "logcnt", "log2phy"):
            assert np.array_equal(got[k][p], getattr(pl, k)), f"{k} plan {p}"
        assert got["steps"][p] == pl.steps


def test_fullsize_overlapped_path_as_benched(dev):
    # the launch configuration the benchmark times on this workload: the 94
    # plans as chunks of 35 and 59 on three streams
    wl = W.get("qwen3_235b")
    P, N = wl.num_plans, wl.pairs_per_plan
    print(f"[fullsize-overlap] {wl.name}: P={P} N={N} chunks 35+59", flush=True)
    ids = W.make_ids(wl, device=dev)
    lay = ep.Layout.from_workload(wl, device=dev)
    load = torch.empty((P, wl.num_experts), dtype=torch.int32, device=dev)
    status = torch.empty(P, dtype=torch.int32, device=dev)
    plan = ep.alloc_plan(P, lay, dev)
    phys = torch.empty_like(ids)
    ep.PathPipeline(lay, P, N, chunks=[35, 59], device=dev).run(ids, load, status, plan, phys)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    del ids
    got = {k: v.cpu().numpy() for k, v in dict(load=load, status=status, phys=phys, quota=plan.phy_quota,
                                                 l2p=plan.log2phy, steps=plan.steps).items()}
    del phys
    torch.cuda.empty_cache()
    lay_o = oracle.Layout.from_workload(wl)
    for p in range(P):
        ld, bad = oracle.histogram(ids_h[p], wl.num_experts)
        assert np.array_equal(got["load"][p], ld), f"load plan {p}"
        pl = oracle.plan(ld, lay_o)
        assert np.array_equal(got["quota"][p], pl.phy_quota), f"quota plan {p}"
        assert np.array_equal(got["l2p"][p], pl.log2phy), f"log2phy plan {p}"
        assert got["steps"][p] == pl.steps
        assert got["status"][p] == (ep.EP_STATUS_STEP_CAP if pl.cap_hit else 0) | (ep.EP_STATUS_BAD_ID if bad else 0)
        ph, _ = oracle.reroute(ids_h[p], wl.num_experts, pl.phy_quota, pl.log2phy, pl.logcnt)
        assert np.array_equal(got["phys"][p], ph), f"reroute plan {p}"
