"""GPU parity of the replica gradient reduction against the CPU oracle, bit-exact
(both fold fp32 gradients over an expert's instances in ascending slot order)."""
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


def _plan(wl, lay_o, plan_index=0, tokens=64):
    wls = wl.scaled(tokens_per_rank=min(wl.tokens_per_rank, tokens), layers=wl.layers, microbatches=wl.microbatches)
    ids = W.make_ids(wls, plans=[plan_index]).numpy()
    return oracle.plan(oracle.histogram(ids[0], wl.num_experts)[0], lay_o)


@pytest.mark.parametrize("name,n", [("tiny", 2048), ("qwen3_235b", 4100), ("deepseek_v3", 1028), ("stress", 4096)])
def test_grad_reduce_matches_oracle(dev, name, n):
    wl = W.get(name)
    lay_o = oracle.Layout.from_workload(wl)
    pl = _plan(wl, lay_o)
    rng = np.random.default_rng(3)
    native = (rng.standard_normal((wl.num_experts, n)) * 10).astype(np.float32)
    slot = (rng.standard_normal((max(lay_o.num_spare, 1), n)) * 10).astype(np.float32)[: lay_o.num_spare]
    lay = ep.Layout.from_workload(wl, device=dev)
    d_native = torch.from_numpy(native).to(dev)
    d_slot = torch.from_numpy(np.ascontiguousarray(slot)).to(dev)
    ep.ep_replica_grad_reduce(d_native, d_slot, torch.from_numpy(pl.log2phy).to(dev),
                              torch.from_numpy(pl.logcnt).to(dev), lay)
    torch.cuda.synchronize()
    ref = native.copy()
    oracle.grad_reduce(ref, slot, lay_o, pl.log2phy, pl.logcnt)
    got = d_native.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(d_slot.cpu().numpy().view(np.uint32), np.ascontiguousarray(slot).view(np.uint32))


def test_grad_reduce_order_by_hand(dev):
    # the fp32 fold in slot order gives 0 where another order would give 1
    lay_o = oracle.Layout.of(3, 3, [1, 1, 1], [1, 0, 2], [1, 0, 1])
    log2phy = np.array([[1, 2, 4], [0, -1, -1], [3, -1, -1]], np.int32)
    logcnt = np.array([3, 1, 1], np.int32)
    native = np.zeros((3, 4), np.float32)
    native[0] = 1.0
    slot = np.array([[1e8] * 4, [-1e8] * 4], np.float32)
    lay = ep.Layout.create(3, [1, 1, 1], [1, 0, 2], [1, 0, 1], device=dev)
    d = torch.from_numpy(native).to(dev)
    ep.ep_replica_grad_reduce(d, torch.from_numpy(slot).to(dev), torch.from_numpy(log2phy).to(dev),
                              torch.from_numpy(logcnt).to(dev), lay)
    torch.cuda.synchronize()
    assert d.cpu().numpy()[0].tolist() == [0.0] * 4


def test_grad_reduce_fullsize_sampled(dev):
    # Qwen3-235B-like layer: 3x4096x1536 fp32 gradient per expert; every element
    # is independent, so sampled windows of every row are folded by the oracle,
    # and every element of every row is compared on the device with the fold
    # written out in slot order (first instance, then + each next instance)
    wl = W.get("qwen3_235b")
    lay_o = oracle.Layout.from_workload(wl)
    pl = _plan(wl, lay_o, tokens=wl.tokens_per_rank)
    n = wl.bytes_per_expert // 2
    lay = ep.Layout.from_workload(wl, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    d_native = torch.randn((wl.num_experts, n), generator=g, device=dev, dtype=torch.float32)
    d_slot = torch.randn((wl.num_spare, n), generator=g, device=dev, dtype=torch.float32)
    starts = [0, 4096 * 17, n // 2 + 12, n - 1024]
    w = 1024
    before_n = [d_native[:, a:a + w].cpu().numpy() for a in starts]
    before_s = [d_slot[:, a:a + w].cpu().numpy() for a in starts]
    # the expected rows of the replicated experts, built before the call
    _, home, _, spare = lay_o.slots()
    ordinal = {int(s): o for o, s in enumerate(spare)}
    expect = {}
    for e in range(wl.num_experts):
        c = int(pl.logcnt[e])
        if c < 2:
            continue
        rows = [d_native[int(home[s])] if home[s] >= 0 else d_slot[ordinal[int(s)]]
                for s in pl.log2phy[e, :c]]
        acc = rows[0].clone()
        for r in rows[1:]:
            acc = acc + r
        expect[e] = acc
    untouched = [e for e in range(wl.num_experts) if e not in expect][:4]
    keep = {e: d_native[e].clone() for e in untouched}
    slot_before = d_slot.clone()
    ep.ep_replica_grad_reduce(d_native, d_slot, torch.from_numpy(pl.log2phy).to(dev),
                              torch.from_numpy(pl.logcnt).to(dev), lay)
    torch.cuda.synchronize()
    assert len(expect) > 10
    for e, acc in expect.items():
        assert torch.equal(d_native[e].view(torch.int32), acc.view(torch.int32)), f"expert {e}"
    for e, row in keep.items():
        assert torch.equal(d_native[e], row), f"expert {e} (one instance) changed"
    assert torch.equal(d_slot, slot_before)
    del expect, keep, slot_before
    for a, bn, bs in zip(starts, before_n, before_s):
        ref = np.ascontiguousarray(bn)
        oracle.grad_reduce(ref, np.ascontiguousarray(bs), lay_o, pl.log2phy, pl.logcnt)
        got = d_native[:, a:a + w].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"window at {a}"
