"""The one-byte ID copy (E <= 256): the histogram stores every pair's ID as a
byte and flags the sub-blocks that hold padding or IDs >= E; the reroute reads
the bytes of unflagged sub-blocks and the int32 IDs of flagged ones.  These
cases mix clean and flagged sub-blocks in one plan, put the largest byte value
(ID 255 at E = 256) in the data, straddle the E = 256 / 257 switch, and feed
IDs that are not 16-byte aligned into an aligned output (the bytes then come
from the histogram's one-pair-per-lane path).  All bit-exact against the CPU
oracle."""
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


def _sub_pairs(N, P, E):
    # the library's sub-block size: about 8192 waves per launch, a power of two
    # from 1024 to 4096, and at least 8 (E + 1) pairs (16 (E + 1) above E = 256)
    want = -(-N * P // 8192)
    lo = max(1024, (8 if E <= 256 else 16) * (E + 1))
    want = max(want, lo)
    sub = 1024
    while sub < want and sub < 4096:
        sub *= 2
    while sub < lo:
        sub *= 2
    return sub


def _layout(E, R=64, spare=1):
    base, extra = divmod(E, R)
    nc = [base + (1 if r < extra else 0) for r in range(R)]
    ne = list(np.random.default_rng(E).permutation(E))
    sc = [spare] * R
    return nc, ne, sc


def _ids(P, N, E, seed):
    # skewed toward the top IDs, so E - 1 (255 at E = 256) is frequent
    rng = np.random.default_rng(seed)
    w = np.arange(1, E + 1, dtype=np.float64) ** 2
    return rng.choice(E, size=(P, N), p=w / w.sum()).astype(np.int32)


def _check(ids_h, E, lay_o, out, disp=None):
    for p in range(ids_h.shape[0]):
        ld, bad = oracle.histogram(ids_h[p], E)
        np.testing.assert_array_equal(out["load"][p].cpu().numpy(), ld, err_msg=f"load plan {p}")
        assert bool(int(out["status"][p]) & ep.EP_STATUS_BAD_ID) == bool(bad)
        r = oracle.plan(ld, lay_o)
        np.testing.assert_array_equal(out["plan"].phy_quota[p].cpu().numpy(), r.phy_quota)
        ph, _ = oracle.reroute(ids_h[p], E, r.phy_quota, r.log2phy, r.logcnt)
        np.testing.assert_array_equal(out["phys"][p].cpu().numpy(), ph, err_msg=f"reroute plan {p}")
        if disp is not None:
            ro, rp, rs, _ = oracle.dispatch(ids_h[p], E, r.phy_quota, r.log2phy, r.logcnt)
            np.testing.assert_array_equal(disp[0][p].cpu().numpy(), ro)
            np.testing.assert_array_equal(disp[1][p].cpu().numpy(), rp)
            np.testing.assert_array_equal(disp[2][p].cpu().numpy(), rs)


@pytest.mark.parametrize("E", [255, 256, 257])
def test_clean_and_flagged_subblocks(dev, E):
    P, N = 3, 100_003          # ragged tail; N % 4 != 0, so plans 1 and 2 are not 16-byte aligned
    print(f"[compact] E={E} P={P} N={N}", flush=True)
    ids_h = _ids(P, N, E, 5 + E)
    sub = _sub_pairs(N, P, E)
    # padding and bad IDs in a few sub-blocks only; plan 1 stays clean
    for p, sb, k, v in [(0, 1, 17, -1), (0, 5, 4000, E), (0, 5, 4001, E + 3), (2, 0, 0, -2),
                        (2, (N - 1) // sub, (N - 1) % sub, -1)]:
        ids_h[p, sb * sub + k] = v
    nc, ne, sc = _layout(E)
    lay_o = oracle.Layout.of(E, 64, nc, ne, sc)
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    ids = torch.from_numpy(ids_h).to(dev)
    out = ep.run_path(ids, lay)
    pl = out["plan"]
    disp = ep.ep_dispatch_layout(ids, lay, pl.phy_quota, pl.log2phy, pl.logcnt, out["ws"])
    torch.cuda.synchronize()
    _check(ids_h, E, lay_o, out, disp)


@pytest.mark.parametrize("N", [16 * 4096, 10 * 4096 + 1500 + 3])
def test_unaligned_ids_aligned_output(dev, N):
    # 4096-pair sub-blocks; N = 10 * 4096 + 1503: a last sub-block of one whole
    # group, one whole tile and a ragged tail; plan 1's rows change alignment
    E, P = 256, 2
    assert _sub_pairs(N, P, E) == 4096
    print(f"[compact] unaligned ids E={E} P={P} N={N}", flush=True)
    ids_h = _ids(P, N, E, 11)
    ids_h[1, 3 * 4096 + 99] = -1
    nc, ne, sc = _layout(E)
    lay_o = oracle.Layout.of(E, 64, nc, ne, sc)
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    # a view one int32 into its buffer: rows 4-byte but not 16-byte aligned
    buf = torch.empty(P * N + 1, dtype=torch.int32, device=dev)
    ids = buf[1:].view(P, N)
    ids.copy_(torch.from_numpy(ids_h))
    assert ids.data_ptr() % 16 != 0
    load, ws, status = ep.ep_load_histogram(ids, lay)
    plan = ep.ep_plan_quota(load, lay, status=status)
    phys = ep.ep_reroute(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws)
    assert phys.data_ptr() % 16 == 0 and ids.data_ptr() % 16 != phys.data_ptr() % 16
    torch.cuda.synchronize()
    _check(ids_h, E, lay_o, dict(load=load, status=status, plan=plan, phys=phys))


def test_byte_copy_and_flags_in_workspace(dev):
    # the workspace layout is internal, but its compact part must hold the IDs'
    # low bytes and one flag per sub-block; read it back through the size formula
    E, P, N = 128, 2, 3 * 4096 + 100
    sub = _sub_pairs(N, P, E)
    assert sub == 2048
    ids_h = _ids(P, N, E, 3)
    ids_h[1, sub + 7] = -1
    nc, ne, sc = _layout(E)
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    ids = torch.from_numpy(ids_h).to(dev)
    _, ws, _ = ep.ep_load_histogram(ids, lay)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()
    stride = (N + 15) // 16 * 16
    got = w[len(w) - P * stride:].reshape(P, stride)[:, :N]
    # within a sub-block, each whole group of 1024 pairs (4 tiles of 64 lanes x
    # 4 pairs) is stored lane-major: byte 16 l + 4 t + k <- pair 256 t + 4 l + k
    want = ids_h.astype(np.uint8).copy()
    for b0 in range(0, N, sub):
        n = min(sub, N - b0)
        for g in range(n // 1024):
            blk = ids_h[:, b0 + 1024 * g: b0 + 1024 * (g + 1)].astype(np.uint8).reshape(P, 4, 64, 4)
            want[:, b0 + 1024 * g: b0 + 1024 * (g + 1)] = blk.transpose(0, 2, 1, 3).reshape(P, 1024)
    np.testing.assert_array_equal(got, want)
    nsb = (N + sub - 1) // sub
    rows = P * (nsb + (nsb + 7) // 8 + 1) * (E + 1) * 4
    f0 = (rows + 255) // 256 * 256
    flags = w[f0:f0 + P * nsb * 4].view(np.int32).reshape(P, nsb)
    want_flags = np.zeros((P, nsb), np.int32)
    want_flags[1, 1] = 1
    np.testing.assert_array_equal(flags, want_flags)


@pytest.mark.parametrize("E", [1, 2, 64])
@pytest.mark.parametrize("N", [1023, 1024, 1025, 2047, 4096 + 3])
def test_small_expert_counts_and_group_edges(dev, E, N):
    # one to a few experts, and plan lengths on both sides of the 1024-pair
    # group and 256-pair tile edges of the byte copy; plan 1 all padding
    P, R = 2, 2 if E < 64 else 16
    rng = np.random.default_rng(E * 7919 + N)
    ids_h = rng.integers(0, E, size=(P, N)).astype(np.int32)
    ids_h[1, :] = -1
    nc = [E - E // 2, E // 2] if R == 2 else [E // R] * R
    ne = list(range(E))
    sc = [1] * R
    lay_o = oracle.Layout.of(E, R, nc, ne, sc)
    lay = ep.Layout.create(E, nc, ne, sc, device=dev)
    ids = torch.from_numpy(ids_h).to(dev)
    out = ep.run_path(ids, lay)
    pl = out["plan"]
    disp = ep.ep_dispatch_layout(ids, lay, pl.phy_quota, pl.log2phy, pl.logcnt, out["ws"])
    torch.cuda.synchronize()
    _check(ids_h, E, lay_o, out, disp)
