"""Launches of many plans give each histogram wave a segment of several
sub-blocks.  This shape (128 plans of 1,100,003 pairs: 4 sub-blocks of 4096
pairs per segment, a last segment of one partial sub-block, odd plan rows
not 16-byte aligned, 1% invalid IDs) checks the histogram, plan, reroute and
dispatch layout of every plan against the CPU oracle, bit-exact."""
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


def _ids(P, N, E, seed):
    rng = np.random.default_rng(seed)
    out = np.empty((P, N), np.int32)
    for p in range(P):
        cdf = np.cumsum(rng.dirichlet(np.full(E, 0.3)))
        out[p] = np.minimum(np.searchsorted(cdf, rng.random(N), side="right"), E - 1)
    return out


def test_segmented_ragged_chain(dev):
    wl = W.get("qwen3_235b")
    E, P, N = wl.num_experts, 128, 1_100_003
    print(f"[segments] P={P} N={N} E={E}", flush=True)
    ids_h = W.inject_invalid(torch.from_numpy(_ids(P, N, E, 77)), E, 0.005, 0.005, seed=78).numpy()
    lay = ep.Layout.from_workload(wl, device=dev)
    ids = torch.from_numpy(ids_h).to(dev)
    out = ep.run_path(ids, lay)
    pl = out["plan"]
    off, pos, src = ep.ep_dispatch_layout(ids, lay, pl.phy_quota, pl.log2phy, pl.logcnt, out["ws"])
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in dict(load=out["load"], status=out["status"], phys=out["phys"],
                                                 quota=pl.phy_quota, l2p=pl.log2phy, off=off, pos=pos,
                                                 src=src).items()}
    del ids, out, off, pos, src
    torch.cuda.empty_cache()
    lay_o = oracle.Layout.from_workload(wl)
    for p in range(P):
        ld, bad = oracle.histogram(ids_h[p], E)
        assert np.array_equal(got["load"][p], ld), f"load plan {p}"
        assert bool(got["status"][p] & ep.EP_STATUS_BAD_ID) == bool(bad), f"status plan {p}"
        r = oracle.plan(ld, lay_o)
        assert np.array_equal(got["quota"][p], r.phy_quota), f"quota plan {p}"
        assert np.array_equal(got["l2p"][p], r.log2phy), f"log2phy plan {p}"
        ph, _ = oracle.reroute(ids_h[p], E, r.phy_quota, r.log2phy, r.logcnt)
        assert np.array_equal(got["phys"][p], ph), f"reroute plan {p}"
        ro, rp, rs, _ = oracle.dispatch(ids_h[p], E, r.phy_quota, r.log2phy, r.logcnt)
        assert np.array_equal(got["off"][p].astype(np.int64), ro), f"slot offsets plan {p}"
        assert np.array_equal(got["pos"][p], rp), f"dispatch_pos plan {p}"
        assert np.array_equal(got["src"][p], rs), f"dispatch_src plan {p}"
