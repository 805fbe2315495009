"""ep_route_noalloc (the histogram -> plan -> reroute chain with the library's
own device scratch instead of a caller workspace) against the same three calls
made with a caller workspace, bit-exact, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input: the scratch
keeps the first call's contents, and the second call's results must not depend
on them.  The oversize batch is rejected on the host before anything runs.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

ep = pytest.importorskip("moe_expert_load_layer_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _reference(ids, lay):
    load, ws, status = ep.ep_load_histogram(ids, lay)
    plan = ep.ep_plan_quota(load, lay, status=status)
    phys = ep.ep_reroute(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws)
    return load, status, plan, phys


def _noalloc(ids, lay, fill):
    P, N = ids.shape
    dev = ids.device
    # outputs pre-filled with junk: every element must be written
    load = torch.full((P, lay.num_experts), fill, dtype=torch.int32, device=dev)
    status = torch.full((P,), fill, dtype=torch.int32, device=dev)
    plan = ep.alloc_plan(P, lay, dev)
    for t in (plan.phy2log, plan.phy_quota, plan.logcnt, plan.log2phy, plan.steps):
        t.fill_(fill)
    phys = torch.full((P, N), fill, dtype=torch.int32, device=dev)
    return ep.ep_route_noalloc(ids, lay, load, status, plan, phys)


def _equal(a, b):
    la, sa, pa, xa = a
    lb, sb, pb, xb = b
    assert torch.equal(la, lb) and torch.equal(sa, sb) and torch.equal(xa, xb)
    for f in ("phy2log", "phy_quota", "logcnt", "log2phy", "steps"):
        assert torch.equal(getattr(pa, f), getattr(pb, f)), f


@pytest.mark.parametrize("name,first,second", [
    ("qwen3_235b", (3, 8192), (1, 1000)),     # one-byte ID copy (E <= 256), two plan sizes
    ("stress", (4, 4096), (2, 777)),          # int32 IDs (E = 384)
    ("glm_4_5", (2, 2048), (1, 5)),
])
def test_noalloc_matches_workspace_calls(dev, name, first, second):
    wl = W.get(name)
    lay = ep.Layout.from_workload(wl, device=dev)
    for k, (P, tokens) in enumerate((first, second)):
        wls = wl.scaled(tokens_per_rank=tokens, layers=min(P, wl.layers),
                        microbatches=max(1, -(-P // wl.layers)))
        ids = W.make_ids(wls, device=dev, plans=list(range(P)))
        if k == 1:
            ids = W.inject_invalid(ids, wl.num_experts, 0.01, 0.002, seed=3)
        print(f"[noalloc] {name} call {k}: P={P} N={ids.shape[1]}", flush=True)
        got = _noalloc(ids, lay, fill=-7 - k)
        ref = _reference(ids, lay)
        torch.cuda.synchronize()
        _equal(got, ref)


def test_noalloc_full_single_layer(dev):
    # one full-size layer of the Qwen3-235B-like workload (4.2M pairs), then a
    # smaller one: the scratch holds up to 14 such plans
    wl = W.get("qwen3_235b")
    lay = ep.Layout.from_workload(wl, device=dev)
    for P, plans in ((2, [0, 1]), (1, [5])):
        ids = W.make_ids(wl, device=dev, plans=plans)
        print(f"[noalloc] qwen3 full size P={P}", flush=True)
        got = _noalloc(ids, lay, fill=-3)
        ref = _reference(ids, lay)
        torch.cuda.synchronize()
        _equal(got, ref)


def test_noalloc_rejects_oversize_batch(dev):
    wl = W.get("qwen3_235b")
    lay = ep.Layout.from_workload(wl, device=dev)
    P, N = 16, wl.pairs_per_plan
    assert ep.ep_workspace_bytes(N, P, wl.num_experts) > ep.EP_NOALLOC_SCRATCH_BYTES
    ids = torch.zeros((P, N), dtype=torch.int32, device=dev)
    load = torch.full((P, wl.num_experts), -5, dtype=torch.int32, device=dev)
    status = torch.zeros(P, dtype=torch.int32, device=dev)
    plan = ep.alloc_plan(P, lay, dev)
    phys = torch.empty_like(ids)
    with pytest.raises(ep.EPBalanceError, match="EP_ERR_TOO_LARGE"):
        ep.ep_route_noalloc(ids, lay, load, status, plan, phys)
    torch.cuda.synchronize()
    assert int((load != -5).sum()) == 0    # nothing ran
