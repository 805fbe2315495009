"""Run-to-run and stream-to-stream determinism of the slot fill, the dispatch
layout and the replica gradient fold: the same inputs give the same bits when a
call is repeated, and when two copies of the call run at once on two streams.
(The histogram, planner, reroute and statistics are covered the same way in the
parity tests.)"""
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


def _plans(wl, dev, plans, tokens):
    wls = wl.scaled(tokens_per_rank=tokens)
    ids = W.make_ids(wls, device=dev, plans=plans)
    lay = ep.Layout.from_workload(wl, device=dev)
    return ids, lay, ep.run_path(ids, lay)


def _two_streams(fn_a, fn_b):
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    start = torch.cuda.Event()
    start.record(torch.cuda.current_stream())
    s1.wait_event(start)
    s2.wait_event(start)
    with torch.cuda.stream(s1):
        fn_a(s1)
    with torch.cuda.stream(s2):
        fn_b(s2)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["qwen3_235b", "stress"])
def test_slot_fill_deterministic(dev, name):
    wl = W.get(name)
    ids, lay, out = _plans(wl, dev, [0], 256)
    # 1.5 MB experts with a ragged last 16 KiB chunk keep the buffers small
    weights = W.make_weights(wl, device=dev, elems_per_expert=3 * 4096 * 64 + 8)
    print(f"[determinism fill] {name} bytes/expert={weights.shape[1] * 2}", flush=True)
    p2l = out["plan"].phy2log[0]
    bufs = [torch.full((wl.num_spare, weights.shape[1]), 3.0, dtype=weights.dtype, device=dev) for _ in range(4)]
    ep.ep_slot_fill(weights, p2l, lay, bufs[0])
    ep.ep_slot_fill(weights, p2l, lay, bufs[1])
    _two_streams(lambda s: ep.ep_slot_fill(weights, p2l, lay, bufs[2], stream=s),
                 lambda s: ep.ep_slot_fill(weights, p2l, lay, bufs[3], stream=s))
    torch.cuda.synchronize()
    for b in bufs[1:]:
        assert torch.equal(b.view(torch.int16), bufs[0].view(torch.int16))
    del weights, bufs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["qwen3_235b", "glm_4_5", "stress"])
def test_dispatch_layout_deterministic(dev, name):
    wl = W.get(name)
    ids, lay, out = _plans(wl, dev, list(range(min(6, wl.num_plans))), 2048)
    print(f"[determinism dispatch] {name} P={ids.shape[0]} N={ids.shape[1]}", flush=True)
    pl = out["plan"]

    def call(stream=None):
        return ep.ep_dispatch_layout(ids, lay, pl.phy_quota, pl.log2phy, pl.logcnt, out["ws"], stream=stream)

    ref = call()
    again = call()
    res = {}
    _two_streams(lambda s: res.__setitem__("a", call(s)), lambda s: res.__setitem__("b", call(s)))
    for got in (again, res["a"], res["b"]):
        for x, y in zip(got, ref):
            assert torch.equal(x, y)


def test_grad_reduce_deterministic(dev):
    wl = W.get("qwen3_235b")
    ids, lay, out = _plans(wl, dev, [3], 1024)
    pl = out["plan"]
    l2p, lc = pl.log2phy[0].contiguous(), pl.logcnt[0].contiguous()
    n = 3 * 4096 * 16
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    native0 = torch.randn((wl.num_experts, n), generator=g, device=dev) * 100
    slot = torch.randn((wl.num_spare, n), generator=g, device=dev)
    print(f"[determinism fold] experts with replicas: {int((lc >= 2).sum())}", flush=True)
    outs = [native0.clone() for _ in range(4)]
    ep.ep_replica_grad_reduce(outs[0], slot, l2p, lc, lay)
    ep.ep_replica_grad_reduce(outs[1], slot, l2p, lc, lay)
    _two_streams(lambda s: ep.ep_replica_grad_reduce(outs[2], slot, l2p, lc, lay, stream=s),
                 lambda s: ep.ep_replica_grad_reduce(outs[3], slot, l2p, lc, lay, stream=s))
    assert int((lc >= 2).sum()) > 0
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))
