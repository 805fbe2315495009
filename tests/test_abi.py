"""The C-ABI library loads on the CPU host and exports every entry point the
public header declares; host-side argument checks run without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep_balance.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(ep_[a-z_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_path():
    names = _declared()
    for n in ("ep_load_histogram", "ep_plan_quota", "ep_reroute", "ep_slot_fill", "ep_balance_stats",
              "ep_slot_fill_workspace_bytes", "ep_sub_block_pairs",
              "ep_workspace_bytes", "ep_layout_init", "ep_layout_table_ints", "ep_status_string",
              "ep_dispatch_layout", "ep_replica_grad_reduce", "ep_route_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import moe_expert_load_layer_amd as ep
    if not os.path.exists(ep.LIB_PATH):
        pytest.skip("library not built")
    lib = ctypes.CDLL(ep.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n


def test_host_side_checks_without_gpu():
    import moe_expert_load_layer_amd as ep
    if not os.path.exists(ep.LIB_PATH):
        pytest.skip("library not built")
    L = ep.lib()
    assert L.ep_status_string(0) == b"EP_OK"
    assert L.ep_status_string(-1) == b"EP_ERR_INVALID_ARG"
    assert L.ep_status_string(-3) == b"EP_ERR_TOO_LARGE"
    assert L.ep_layout_table_ints(12, 8, 4) == 2 * 8 + 1 + 3 * 16 + 12 + 4
    assert L.ep_workspace_bytes(-1, 1, 4) == 0
    assert L.ep_workspace_bytes(0, 3, 4) == 3 * 1 * 5 * 4      # only the per-plan totals row
    # workspace grows with the number of sub-blocks: count rows of E + 1 ints
    a = L.ep_workspace_bytes(1 << 20, 1, 300)
    b = L.ep_workspace_bytes(1 << 21, 1, 300)
    assert 0 < a < b
    assert a % (301 * 4) == 0
    # E <= 256 adds the one-byte copy of the IDs and a flag per sub-block; the
    # count table stays under 1/2 byte per pair
    c = L.ep_workspace_bytes(1 << 20, 1, 256)
    assert (1 << 20) < c < (1 << 20) * 3 // 2 + 4096
    assert L.ep_workspace_bytes(1000, 2, 8) >= 2 * 1008
    # null pointers are rejected before any device work
    lay = ep._CLayout(12, 8, 16, 4, 5, 2, 1, 0, None)
    rc = L.ep_load_histogram(None, 512, 1, ctypes.byref(lay), None, None, 0, None, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    rc = L.ep_plan_quota(None, 1, ctypes.byref(lay), None, None, None, None, None, None, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    # inconsistent layout header (rho must be min(R, 1+S)) is rejected
    lay_bad = ep._CLayout(12, 8, 16, 4, 4, 2, 1, 0, ctypes.c_void_p(16))
    rc = L.ep_balance_stats(ctypes.c_void_p(16), ctypes.c_void_p(16), 1, ctypes.byref(lay_bad),
                            ctypes.c_void_p(16), ctypes.c_void_p(16), None, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    # slot fill needs a multiple of 16 bytes per expert
    lay_ok = ep._CLayout(12, 8, 16, 4, 5, 2, 1, 0, ctypes.c_void_p(16))
    rc = L.ep_slot_fill(ctypes.c_void_p(16), 24, ctypes.c_void_p(16), ctypes.byref(lay_ok),
                        ctypes.c_void_p(16), None, 0, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    # its optional fill-list workspace: 3 int32 values per spare slot (item
    # expert, item start, target) and two more (item count, end of the last
    # item); a smaller or misaligned one is rejected
    assert L.ep_slot_fill_workspace_bytes(ctypes.byref(lay_ok)) == (3 * 4 + 2) * 4
    rc = L.ep_slot_fill(ctypes.c_void_p(16), 32, ctypes.c_void_p(16), ctypes.byref(lay_ok),
                        ctypes.c_void_p(16), ctypes.c_void_p(64), 55, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    rc = L.ep_slot_fill(ctypes.c_void_p(16), 32, ctypes.c_void_p(16), ctypes.byref(lay_ok),
                        ctypes.c_void_p(16), ctypes.c_void_p(72), 56, None)
    assert rc == ep.EP_ERR_INVALID_ARG


def test_layout_init_rejects_bad_placement_on_host():
    import moe_expert_load_layer_amd as ep
    if not os.path.exists(ep.LIB_PATH):
        pytest.skip("library not built")
    L = ep.lib()
    nc = (ctypes.c_int32 * 2)(1, 1)
    ne = (ctypes.c_int32 * 2)(0, 0)          # expert 0 twice, expert 1 missing
    sc = (ctypes.c_int32 * 2)(0, 1)
    buf = (ctypes.c_int32 * 64)()
    out = ep._CLayout()
    rc = L.ep_layout_init(2, 2, ctypes.cast(nc, ctypes.c_void_p), ctypes.cast(ne, ctypes.c_void_p),
                          ctypes.cast(sc, ctypes.c_void_p), ctypes.cast(buf, ctypes.c_void_p), 64,
                          ctypes.byref(out))
    assert rc == ep.EP_ERR_INVALID_ARG


def test_entry_points_reject_unsupported_shapes_on_host():
    import moe_expert_load_layer_amd as ep
    if not os.path.exists(ep.LIB_PATH):
        pytest.skip("library not built")
    L = ep.lib()
    fake = ctypes.c_void_p(256)
    # rho = min(R, 1 + S) = 100 > 64: the gradient fold keeps at most 64 rows
    wide = ep._CLayout(100, 100, 200, 100, 100, 1, 1, 0, fake)
    rc = L.ep_replica_grad_reduce(fake, 64, fake, fake, fake, ctypes.byref(wide), None)
    assert rc == ep.EP_ERR_INVALID_ARG
    rc = L.ep_plan_quota(fake, 1, ctypes.byref(wide), fake, fake, fake, fake, None, None, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    # a negative domain size is not a layout
    bad_dom = ep._CLayout(12, 8, 16, 4, 5, 2, 1, -1, fake)
    rc = L.ep_plan_quota(fake, 1, ctypes.byref(bad_dom), fake, fake, fake, fake, None, None, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    # the dispatch layout needs 4-byte aligned outputs
    lay = ep._CLayout(12, 8, 16, 4, 5, 2, 1, 0, fake)
    ws = L.ep_workspace_bytes(512, 1, 12)
    rc = L.ep_dispatch_layout(fake, 512, 1, ctypes.byref(lay), fake, fake, fake, fake, ws, fake,
                              ctypes.c_void_p(258), fake, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    rc = L.ep_dispatch_layout(fake, 512, 1, ctypes.byref(lay), fake, fake, fake, fake, ws,
                              ctypes.c_void_p(257), fake, fake, None)
    assert rc == ep.EP_ERR_INVALID_ARG
    # gradient rows must be a multiple of 4 floats
    rc = L.ep_replica_grad_reduce(fake, 6, fake, fake, fake, ctypes.byref(lay), None)
    assert rc == ep.EP_ERR_INVALID_ARG


def test_sub_block_query_matches_the_workspace():
    # ep_sub_block_pairs (which the bench uses to count the histogram's count
    # rows) and ep_workspace_bytes agree on the geometry
    import moe_expert_load_layer_amd as ep
    if not os.path.exists(ep.LIB_PATH):
        pytest.skip("library not built")
    a = lambda x: (x + 255) // 256 * 256
    for N, P, E in [(4194304, 256, 384), (4194304, 94, 300), (100003, 3, 257), (1 << 20, 1, 300),
                    (5, 2, 1000), (4194304, 94, 128), (2097152, 58, 256), (5242880, 92, 160),
                    (4194304, 47, 128), (1000, 1, 12)]:
        sub = ep.ep_sub_block_pairs(N, P, E)
        assert sub >= 1024 and sub & (sub - 1) == 0
        nsb = -(-N // sub)
        nseg = -(-nsb // 8)
        rows = P * (nsb + nseg + 1) * (E + 1) * 4
        want = a(rows) + a(P * nsb * 4) + P * ((N + 15) // 16 * 16) if E <= 256 else rows
        assert ep.ep_workspace_bytes(N, P, E) == want, (N, P, E)


def test_noalloc_host_checks_without_gpu():
    # a batch whose workspace exceeds the library's scratch is refused on the
    # host (before any HIP call), and so is a missing layout
    import moe_expert_load_layer_amd as ep
    if not os.path.exists(ep.LIB_PATH):
        pytest.skip("library not built")
    L = ep.lib()
    lay = ep._CLayout(128, 64, 192, 64, 64, 2, 1, 0, None)
    N, P = 64 * 8192 * 8, 16
    assert L.ep_workspace_bytes(N, P, 128) > ep.EP_NOALLOC_SCRATCH_BYTES
    nul = [None] * 8
    assert L.ep_route_noalloc(None, N, P, ctypes.byref(lay), *nul, None) == ep.EP_ERR_TOO_LARGE
    assert L.ep_route_noalloc(None, N, 1, None, *nul, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_route_noalloc(None, -1, 1, ctypes.byref(lay), *nul, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_route_noalloc(None, N, 70000, ctypes.byref(lay), *nul, None) == ep.EP_ERR_INVALID_ARG


def test_sub_block_geometry():
    # the sub-block sizes the launches use: about 8192 waves per launch, at
    # least 8 (E + 1) pairs with E <= 256 and 16 (E + 1) above, 1024..4096
    # unless that bound asks for more
    import moe_expert_load_layer_amd as ep
    if not os.path.exists(ep.LIB_PATH):
        pytest.skip("library not built")
    assert ep.ep_sub_block_pairs(4194304, 94, 128) == 4096     # 94 Qwen3-like plans
    assert ep.ep_sub_block_pairs(4194304, 1, 128) == 2048      # one such plan
    assert ep.ep_sub_block_pairs(2097152, 58, 256) == 4096     # DeepSeek-V3-like batch
    assert ep.ep_sub_block_pairs(4194304, 256, 384) == 8192    # stress batch
    assert ep.ep_sub_block_pairs(512, 2, 12) == 1024
    assert ep.ep_sub_block_pairs(-1, 1, 12) == 0
    # the count rows: one row of E + 1 int32 per sub-block, plus segment rows
    N, P, E = 4194304, 94, 128
    sub = ep.ep_sub_block_pairs(N, P, E)
    nsb = -(-N // sub)
    nseg = -(-nsb // 8)
    rows = P * (nsb + nseg + 1) * (E + 1) * 4
    assert ep.ep_workspace_bytes(N, P, E) >= rows + P * N


def test_pipelined_route_host_checks_without_gpu():
    # the overlapped chain refuses bad chunkings and stream sets on the host,
    # before any HIP call
    import moe_expert_load_layer_amd as ep
    if not os.path.exists(ep.LIB_PATH):
        pytest.skip("library not built")
    L = ep.lib()
    i32 = ctypes.c_int32
    sizes = (i32 * 2)(3, 4)
    E, N = 12, 1000
    one = L.ep_workspace_bytes(N, 3, E)
    two = L.ep_workspace_bytes(N, 4, E)
    r256 = lambda x: (x + 255) // 256 * 256
    assert L.ep_pipeline_workspace_bytes(N, sizes, 2, E) == r256(one) + r256(two)
    assert L.ep_pipeline_workspace_bytes(N, sizes, 17, E) == 0          # more than EP_MAX_CHUNKS
    lay = ep._CLayout(12, 8, 16, 4, 5, 2, 1, 0, ctypes.c_void_p(16))
    fake = ctypes.c_void_p(4096)
    ev = (ctypes.c_void_p * 6)(*([4096] * 6))
    def args(P, ch, n, s0, side):
        arr = (ctypes.c_void_p * 3)(*side) if side is not None else None
        return L.ep_route_pipelined(fake, N, P, ctypes.byref(lay), ch, n, fake, fake, fake, fake, fake, fake, None,
                                    fake, fake, 1 << 20, s0, arr, ev)
    s_a, s_b, s_c = 8, 24, 40
    assert args(8, sizes, 2, None, (s_a, s_b, s_c)) == ep.EP_ERR_INVALID_ARG   # chunks sum to 7, not 8
    assert args(7, sizes, 2, None, (s_a, s_b, s_a)) == ep.EP_ERR_INVALID_ARG   # one side stream twice
    assert args(7, sizes, 2, s_b, (s_a, s_b, s_c)) == ep.EP_ERR_INVALID_ARG    # side stream = caller's
    assert args(7, sizes, 2, None, (s_a, None, s_c)) == ep.EP_ERR_INVALID_ARG  # missing side stream
    assert args(7, sizes, 2, None, None) == ep.EP_ERR_INVALID_ARG              # no side streams
    assert args(7, sizes, 0, None, (s_a, s_b, s_c)) == ep.EP_ERR_INVALID_ARG   # no chunk
