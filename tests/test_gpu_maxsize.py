"""The largest plan the boundary admits: N = 2^31 - 99 pairs in one plan (the
pair index and every position still fit int32; offsets and loops must not).
Skewed routing over 64 experts on 16 ranks, with padding and invalid IDs, a
ragged last sub-block; histogram, plan, reroute and dispatch layout are
compared with the CPU oracle element by element."""
import time

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

ep = pytest.importorskip("moe_expert_load_layer_amd")

E, R = 64, 16
N = (1 << 31) - 99


def _say(msg):
    print(f"[maxsize {time.strftime('%H:%M:%S')}] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info()
    if free < 60 * (1 << 30):
        pytest.skip("needs 60 GiB of free device memory")
    return torch.device("cuda:0")


def _ids(dev):
    rng = np.random.default_rng(20260107)
    cdf = torch.from_numpy(np.cumsum(rng.dirichlet(np.full(E, 0.3)))).to(dev, torch.float32)
    cdf[-1] = 2.0                                       # every draw lands in [0, E)
    g = torch.Generator(device=dev)
    g.manual_seed(20260107)
    ids = torch.empty(N, dtype=torch.int32, device=dev)
    step = 1 << 28
    for a in range(0, N, step):
        b = min(N, a + step)
        u = torch.rand(b - a, generator=g, device=dev)
        ids[a:b] = torch.searchsorted(cdf, u, right=True, out_int32=True)
    ids[::997] = -1                                     # padding
    ids[5::100003] = E + 5                              # invalid IDs
    return ids.view(1, N)


def test_max_pairs_per_plan(dev):
    _say(f"N={N} E={E} R={R}: generating IDs")
    ids = _ids(dev)
    nc = [E // R] * R
    ne = list(range(E))
    sc = [1] * R
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    _say("histogram, plan, reroute, dispatch layout on the GPU")
    load, ws, status = ep.ep_load_histogram(ids, lay)
    plan = ep.ep_plan_quota(load, lay, status=status)
    phys = ep.ep_reroute(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws)
    off, pos, src = ep.ep_dispatch_layout(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws)
    torch.cuda.synchronize()
    _say("copying to the host")
    ids_h = ids[0].cpu().numpy()
    g = dict(load=load[0].cpu().numpy(), status=int(status[0]), quota=plan.phy_quota[0].cpu().numpy(),
             l2p=plan.log2phy[0].cpu().numpy(), off=off[0].cpu().numpy())
    del ids, ws, load, status
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    _say("oracle histogram and plan")
    ld, bad = oracle.histogram(ids_h, E)
    assert bad > 0
    assert np.array_equal(g["load"], ld)
    assert g["status"] & ep.EP_STATUS_BAD_ID
    pl = oracle.plan(ld, lay_o)
    assert np.array_equal(g["quota"], pl.phy_quota)
    assert np.array_equal(g["l2p"], pl.log2phy)
    _say("oracle reroute")
    ph, _ = oracle.reroute(ids_h, E, pl.phy_quota, pl.log2phy, pl.logcnt)
    assert np.array_equal(phys[0].cpu().numpy(), ph)
    del phys, ph
    torch.cuda.empty_cache()
    _say("oracle dispatch layout")
    ro, rp, rs, _ = oracle.dispatch(ids_h, E, pl.phy_quota, pl.log2phy, pl.logcnt)
    assert np.array_equal(g["off"].astype(np.int64), ro)
    assert np.array_equal(pos[0].cpu().numpy(), rp)
    del rp
    assert np.array_equal(src[0].cpu().numpy(), rs)
    _say("done")
