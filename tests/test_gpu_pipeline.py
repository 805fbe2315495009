"""The overlapped path (chunks of plans on three streams) gives the oracle's
histogram, plans and rerouted IDs for every plan, for any number of chunks."""
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


@pytest.mark.parametrize("chunks", [1, 2, 3, 7, 50])
def test_pipeline_matches_oracle(dev, chunks):
    wl = W.get("qwen3_235b")
    wls = wl.scaled(tokens_per_rank=97, layers=7, microbatches=1)
    ids_h = W.inject_invalid(W.make_ids(wls), wl.num_experts, 0.01, 0.005).numpy()
    P, N = ids_h.shape
    print(f"[pipeline] chunks={chunks} P={P} N={N}", flush=True)
    lay = ep.Layout.from_workload(wl, device=dev)
    ids = torch.from_numpy(ids_h).to(dev)
    load = torch.full((P, wl.num_experts), -7, dtype=torch.int32, device=dev)
    status = torch.full((P,), -7, dtype=torch.int32, device=dev)
    plan = ep.alloc_plan(P, lay, dev)
    phys = torch.full_like(ids, -7)
    pipe = ep.PathPipeline(lay, P, N, chunks=chunks, device=dev)
    for rep in range(2):            # the second run reuses streams, events and workspaces
        pipe.run(ids, load, status, plan, phys)
        torch.cuda.synchronize()
        lay_o = oracle.Layout.from_workload(wl)
        for p in range(P):
            ld, bad = oracle.histogram(ids_h[p], wl.num_experts)
            assert np.array_equal(load[p].cpu().numpy(), ld), f"load plan {p} rep {rep}"
            assert int(status[p]) == (ep.EP_STATUS_BAD_ID if bad else 0)
            r = oracle.plan(ld, lay_o)
            assert np.array_equal(plan.phy2log[p].cpu().numpy(), r.phy2log)
            assert np.array_equal(plan.phy_quota[p].cpu().numpy(), r.phy_quota)
            assert np.array_equal(plan.log2phy[p].cpu().numpy(), r.log2phy)
            ph, _ = oracle.reroute(ids_h[p], wl.num_experts, r.phy_quota, r.log2phy, r.logcnt)
            assert np.array_equal(phys[p].cpu().numpy(), ph), f"reroute plan {p} rep {rep}"
        phys.fill_(-7)
        load.fill_(-7)


def test_pipeline_rejects_other_shapes(dev):
    wl = W.get("tiny")
    lay = ep.Layout.from_workload(wl, device=dev)
    pipe = ep.PathPipeline(lay, 2, 64, chunks=2, device=dev)
    ids = torch.zeros((2, 65), dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        pipe.run(ids, None, None, None, None)


def test_pipeline_uneven_sizes_and_bad_split(dev):
    wl = W.get("tiny")
    wls = wl.scaled(layers=2, microbatches=3)
    ids_h = W.make_ids(wls).numpy()
    P, N = ids_h.shape
    lay = ep.Layout.from_workload(wl, device=dev)
    with pytest.raises(ValueError):
        ep.PathPipeline(lay, P, N, chunks=[1, P], device=dev)
    ids = torch.from_numpy(ids_h).to(dev)
    load = torch.empty((P, wl.num_experts), dtype=torch.int32, device=dev)
    status = torch.empty(P, dtype=torch.int32, device=dev)
    plan = ep.alloc_plan(P, lay, dev)
    phys = torch.empty_like(ids)
    ep.PathPipeline(lay, P, N, chunks=[1, P - 1], device=dev).run(ids, load, status, plan, phys)
    torch.cuda.synchronize()
    lay_o = oracle.Layout.from_workload(wl)
    for p in range(P):
        ld, _ = oracle.histogram(ids_h[p], wl.num_experts)
        r = oracle.plan(ld, lay_o)
        ph, _ = oracle.reroute(ids_h[p], wl.num_experts, r.phy_quota, r.log2phy, r.logcnt)
        assert np.array_equal(phys[p].cpu().numpy(), ph)
