"""Python binding of the gfx950 HIP library ``libepbalance.so`` (C ABI in include/ep_balance.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step runs in the library's kernels.  Function names match the C
entry points.  Importing this module does not touch the GPU; the first call
loads the library and raises :class:`EPBalanceError` if it is missing (no CPU
fallback exists).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libepbalance.so")

EP_OK = 0
EP_ERR_INVALID_ARG = -1
EP_ERR_HIP = -2
EP_ERR_TOO_LARGE = -3
EP_NOALLOC_SCRATCH_BYTES = 64 << 20
EP_STATUS_BAD_ID = 1
EP_STATUS_STEP_CAP = 2
EP_STATUS_BAD_LOAD = 4


class EPBalanceError(RuntimeError):
    pass


class _CLayout(ctypes.Structure):
    _fields_ = [
        ("num_experts", ctypes.c_int32),
        ("num_ranks", ctypes.c_int32),
        ("num_phys", ctypes.c_int32),
        ("num_spare", ctypes.c_int32),
        ("max_replicas", ctypes.c_int32),
        ("max_rank_natives", ctypes.c_int32),
        ("max_rank_spares", ctypes.c_int32),
        ("ranks_per_domain", ctypes.c_int32),
        ("tables", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise EPBalanceError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lp = ctypes.POINTER(_CLayout)
        L.ep_layout_table_ints.argtypes = [i32, i32, i32]
        L.ep_layout_table_ints.restype = sz
        L.ep_layout_init.argtypes = [i32, i32, vp, vp, vp, vp, sz, lp]
        L.ep_workspace_bytes.argtypes = [i64, i32, i32]
        L.ep_workspace_bytes.restype = sz
        L.ep_sub_block_pairs.argtypes = [i64, i32, i32]
        L.ep_sub_block_pairs.restype = i64
        L.ep_load_histogram.argtypes = [vp, i64, i32, lp, vp, vp, sz, vp, vp]
        L.ep_plan_quota.argtypes = [vp, i32, lp, vp, vp, vp, vp, vp, vp, vp]
        L.ep_reroute.argtypes = [vp, i64, i32, lp, vp, vp, vp, vp, sz, vp, vp]
        L.ep_slot_fill.argtypes = [vp, i64, vp, lp, vp, vp, sz, vp]
        L.ep_slot_fill_workspace_bytes.argtypes = [lp]
        L.ep_slot_fill_workspace_bytes.restype = sz
        L.ep_dispatch_layout.argtypes = [vp, i64, i32, lp, vp, vp, vp, vp, sz, vp, vp, vp, vp]
        L.ep_replica_grad_reduce.argtypes = [vp, i64, vp, vp, vp, lp, vp]
        L.ep_balance_stats.argtypes = [vp, vp, i32, lp, vp, vp, vp, vp]
        L.ep_route_noalloc.argtypes = [vp, i64, i32, lp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.ep_pipeline_workspace_bytes.argtypes = [i64, ctypes.POINTER(i32), i32, i32]
        L.ep_pipeline_workspace_bytes.restype = sz
        L.ep_route_pipelined.argtypes = [vp, i64, i32, lp, ctypes.POINTER(i32), i32, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, sz, vp, ctypes.POINTER(vp), ctypes.POINTER(vp)]
        L.ep_status_string.argtypes = [ctypes.c_int]
        L.ep_status_string.restype = ctypes.c_char_p
        for f in ("ep_layout_init", "ep_load_histogram", "ep_plan_quota", "ep_reroute",
                  "ep_slot_fill", "ep_balance_stats", "ep_dispatch_layout", "ep_replica_grad_reduce",
                  "ep_route_noalloc", "ep_route_pipelined"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != EP_OK:
        raise EPBalanceError(f"{what}: {lib().ep_status_string(rc).decode()} ({rc})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise EPBalanceError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise EPBalanceError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise EPBalanceError(f"{name} must be contiguous")
    return t


def _arg(t: Optional[torch.Tensor], dtype: torch.dtype, shape, name: str) -> torch.Tensor:
    """A device tensor of exactly this dtype and shape: the kernels trust the sizes."""
    if t is None:
        raise EPBalanceError(f"{name} is required")
    _dev(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise EPBalanceError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ids(t: torch.Tensor, name: str = "topk_ids"):
    _dev(t, torch.int32, name)
    if t.dim() != 2:
        raise EPBalanceError(f"{name} must be [plans][pairs], got shape {tuple(t.shape)}")
    return t.shape


def _ws(ws: torch.Tensor, N: int, P: int, layout: "Layout") -> torch.Tensor:
    if not (ws.is_cuda and ws.is_contiguous()):
        raise EPBalanceError("ws must be a contiguous device tensor")
    if ws.numel() * ws.element_size() < ep_workspace_bytes(N, P, layout.num_experts):
        raise EPBalanceError("ws is smaller than ep_workspace_bytes(N, P, E)")
    return ws


def _plan_args(layout: "Layout", P: int, phy_quota, log2phy, logcnt):
    E, Phi, rho = layout.num_experts, layout.num_phys, layout.max_replicas
    _arg(phy_quota, torch.int32, (P, Phi), "phy_quota")
    _arg(log2phy, torch.int32, (P, E, rho), "log2phy")
    _arg(logcnt, torch.int32, (P, E), "logcnt")


def _stream(stream: Optional[torch.cuda.Stream]):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class Layout:
    """Native placement + spare slots of one EP group, with its device tables."""

    num_experts: int
    num_ranks: int
    num_phys: int
    num_spare: int
    max_replicas: int
    tables: torch.Tensor
    c: _CLayout

    @classmethod
    def create(cls, num_experts: int, native_count: Sequence[int], native_experts: Sequence[int],
               spare_count: Sequence[int], device="cuda") -> "Layout":
        R = len(native_count)
        nc = (ctypes.c_int32 * R)(*[int(x) for x in native_count])
        ne = (ctypes.c_int32 * len(native_experts))(*[int(x) for x in native_experts])
        sc = (ctypes.c_int32 * R)(*[int(x) for x in spare_count])
        S = int(sum(int(x) for x in spare_count))
        n = lib().ep_layout_table_ints(num_experts, R, S)
        if n == 0:
            raise EPBalanceError("invalid layout sizes")
        tables = torch.empty(n, dtype=torch.int32, device=device)
        c = _CLayout()
        rc = lib().ep_layout_init(num_experts, R, ctypes.cast(nc, ctypes.c_void_p),
                                  ctypes.cast(ne, ctypes.c_void_p), ctypes.cast(sc, ctypes.c_void_p),
                                  _ptr(tables), n, ctypes.byref(c))
        _check(rc, "ep_layout_init")
        return cls(c.num_experts, c.num_ranks, c.num_phys, c.num_spare, c.max_replicas, tables, c)

    @classmethod
    def from_workload(cls, wl, device="cuda") -> "Layout":
        return cls.create(wl.num_experts, wl.native_count, list(wl.native_experts()), wl.spare_count,
                          device)

    def ref(self):
        return ctypes.byref(self.c)

    def with_domain(self, ranks_per_domain: int) -> "Layout":
        """The same layout with replicas confined to domains of that many ranks (0: anywhere)."""
        c = _CLayout.from_buffer_copy(self.c)
        c.ranks_per_domain = int(ranks_per_domain)
        return Layout(self.num_experts, self.num_ranks, self.num_phys, self.num_spare, self.max_replicas,
                      self.tables, c)


def ep_workspace_bytes(pairs_per_plan: int, num_plans: int, num_experts: int) -> int:
    return int(lib().ep_workspace_bytes(pairs_per_plan, num_plans, num_experts))


def ep_sub_block_pairs(pairs_per_plan: int, num_plans: int, num_experts: int) -> int:
    return int(lib().ep_sub_block_pairs(int(pairs_per_plan), int(num_plans), int(num_experts)))


def workspace(topk_ids: torch.Tensor, layout: Layout) -> torch.Tensor:
    P, N = topk_ids.shape
    nbytes = ep_workspace_bytes(N, P, layout.num_experts)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=topk_ids.device)


def ep_load_histogram(topk_ids: torch.Tensor, layout: Layout, load=None, ws=None, status=None,
                      stream=None):
    """topk_ids int32 [P][N] -> (load int32 [P][E], ws, status uint32-as-int32 [P])."""
    P, N = _ids(topk_ids)
    dev = topk_ids.device
    load = torch.empty((P, layout.num_experts), dtype=torch.int32, device=dev) if load is None else load
    ws = workspace(topk_ids, layout) if ws is None else _ws(ws, N, P, layout)
    status = torch.empty(P, dtype=torch.int32, device=dev) if status is None else status
    _arg(load, torch.int32, (P, layout.num_experts), "load"); _arg(status, torch.int32, (P,), "status")
    rc = lib().ep_load_histogram(_ptr(topk_ids), N, P, layout.ref(), _ptr(load), _ptr(ws),
                                 ws.numel() * ws.element_size(), _ptr(status), _stream(stream))
    _check(rc, "ep_load_histogram")
    return load, ws, status


@dataclass
class PlanOut:
    phy2log: torch.Tensor    # int32 [P][Phi]
    phy_quota: torch.Tensor  # int32 [P][Phi]
    logcnt: torch.Tensor     # int32 [P][E]
    log2phy: torch.Tensor    # int32 [P][E][rho]
    steps: torch.Tensor      # int32 [P]


def alloc_plan(P: int, layout: Layout, device) -> PlanOut:
    E, Phi, rho = layout.num_experts, layout.num_phys, layout.max_replicas
    return PlanOut(torch.empty((P, Phi), dtype=torch.int32, device=device),
                   torch.empty((P, Phi), dtype=torch.int32, device=device),
                   torch.empty((P, E), dtype=torch.int32, device=device),
                   torch.empty((P, E, rho), dtype=torch.int32, device=device),
                   torch.empty(P, dtype=torch.int32, device=device))


def ep_plan_quota(load: torch.Tensor, layout: Layout, out: Optional[PlanOut] = None, status=None,
                  stream=None) -> PlanOut:
    _dev(load, torch.int32, "load")
    P = load.shape[0]
    _arg(load, torch.int32, (P, layout.num_experts), "load")
    out = alloc_plan(P, layout, load.device) if out is None else out
    _arg(out.phy2log, torch.int32, (P, layout.num_phys), "phy2log")
    _plan_args(layout, P, out.phy_quota, out.log2phy, out.logcnt)
    _arg(out.steps, torch.int32, (P,), "steps")
    if status is not None:
        _arg(status, torch.int32, (P,), "status")
    rc = lib().ep_plan_quota(_ptr(load), P, layout.ref(), _ptr(out.phy2log), _ptr(out.phy_quota),
                             _ptr(out.logcnt), _ptr(out.log2phy), _ptr(out.steps), _ptr(status),
                             _stream(stream))
    _check(rc, "ep_plan_quota")
    return out


def ep_reroute(topk_ids: torch.Tensor, layout: Layout, phy_quota: torch.Tensor, log2phy: torch.Tensor,
               logcnt: torch.Tensor, ws: torch.Tensor, phys_ids=None, stream=None) -> torch.Tensor:
    P, N = _ids(topk_ids)
    _plan_args(layout, P, phy_quota, log2phy, logcnt)
    _ws(ws, N, P, layout)
    phys_ids = torch.empty_like(topk_ids) if phys_ids is None else _arg(phys_ids, torch.int32, (P, N), "phys_ids")
    rc = lib().ep_reroute(_ptr(topk_ids), N, P, layout.ref(), _ptr(phy_quota), _ptr(log2phy),
                          _ptr(logcnt), _ptr(ws), ws.numel() * ws.element_size(), _ptr(phys_ids),
                          _stream(stream))
    _check(rc, "ep_reroute")
    return phys_ids


def ep_dispatch_layout(topk_ids: torch.Tensor, layout: Layout, phy_quota: torch.Tensor,
                       log2phy: torch.Tensor, logcnt: torch.Tensor, ws: torch.Tensor, slot_offsets=None,
                       dispatch_pos=None, dispatch_src=None, stream=None):
    """-> (slot_offsets int32 [P][Phi+1], dispatch_pos int32 [P][N], dispatch_src int32 [P][N])."""
    P, N = _ids(topk_ids)
    _plan_args(layout, P, phy_quota, log2phy, logcnt)
    _ws(ws, N, P, layout)
    dev = topk_ids.device
    if slot_offsets is None:
        slot_offsets = torch.empty((P, layout.num_phys + 1), dtype=torch.int32, device=dev)
    _arg(slot_offsets, torch.int32, (P, layout.num_phys + 1), "slot_offsets")
    dispatch_pos = torch.empty_like(topk_ids) if dispatch_pos is None else dispatch_pos
    dispatch_src = torch.empty_like(topk_ids) if dispatch_src is None else dispatch_src
    _arg(dispatch_pos, torch.int32, (P, N), "dispatch_pos"); _arg(dispatch_src, torch.int32, (P, N), "dispatch_src")
    rc = lib().ep_dispatch_layout(_ptr(topk_ids), N, P, layout.ref(), _ptr(phy_quota), _ptr(log2phy),
                                  _ptr(logcnt), _ptr(ws), ws.numel() * ws.element_size(),
                                  _ptr(slot_offsets), _ptr(dispatch_pos), _ptr(dispatch_src),
                                  _stream(stream))
    _check(rc, "ep_dispatch_layout")
    return slot_offsets, dispatch_pos, dispatch_src


def ep_replica_grad_reduce(native_grads: torch.Tensor, slot_grads: torch.Tensor, log2phy: torch.Tensor,
                           logcnt: torch.Tensor, layout: Layout, stream=None) -> torch.Tensor:
    """native_grads float32 [E][n] (in place), slot_grads float32 [S][n], one plan's log2phy/logcnt."""
    _dev(native_grads, torch.float32, "native_grads")
    if native_grads.dim() != 2 or native_grads.shape[0] != layout.num_experts:
        raise EPBalanceError(f"native_grads must be [E][n] with E = {layout.num_experts}")
    n = native_grads.shape[1]
    _arg(log2phy, torch.int32, (layout.num_experts, layout.max_replicas), "log2phy")
    _arg(logcnt, torch.int32, (layout.num_experts,), "logcnt")
    if layout.num_spare:
        _arg(slot_grads, torch.float32, (layout.num_spare, n), "slot_grads")
    rc = lib().ep_replica_grad_reduce(_ptr(native_grads), n, _ptr(slot_grads) if layout.num_spare else None,
                                      _ptr(log2phy), _ptr(logcnt), layout.ref(), _stream(stream))
    _check(rc, "ep_replica_grad_reduce")
    return native_grads


def ep_route_noalloc(topk_ids: torch.Tensor, layout: Layout, load: torch.Tensor, status: torch.Tensor,
                     plan: PlanOut, phys_ids: torch.Tensor, stream=None):
    """hist -> plan -> reroute in one call that allocates nothing: the workspace is
    the library's own device array (EP_NOALLOC_SCRATCH_BYTES per GPU).  Every
    output is the caller's; calls that overlap on one GPU race."""
    P, N = _ids(topk_ids)
    _arg(load, torch.int32, (P, layout.num_experts), "load"); _arg(status, torch.int32, (P,), "status")
    _arg(plan.phy2log, torch.int32, (P, layout.num_phys), "phy2log")
    _plan_args(layout, P, plan.phy_quota, plan.log2phy, plan.logcnt)
    _arg(plan.steps, torch.int32, (P,), "steps")
    _arg(phys_ids, torch.int32, (P, N), "phys_ids")
    rc = lib().ep_route_noalloc(_ptr(topk_ids), N, P, layout.ref(), _ptr(load), _ptr(status),
                                _ptr(plan.phy2log), _ptr(plan.phy_quota), _ptr(plan.logcnt),
                                _ptr(plan.log2phy), _ptr(plan.steps), _ptr(phys_ids), _stream(stream))
    _check(rc, "ep_route_noalloc")
    return load, status, plan, phys_ids


def ep_slot_fill_workspace_bytes(layout: Layout) -> int:
    return int(lib().ep_slot_fill_workspace_bytes(layout.ref()))


def slot_fill_workspace(layout: Layout, device) -> torch.Tensor:
    """A workspace for ep_slot_fill (reusable by consecutive calls on one stream)."""
    return torch.empty(max(ep_slot_fill_workspace_bytes(layout), 16), dtype=torch.uint8, device=device)


def ep_slot_fill(expert_weights: torch.Tensor, phy2log: torch.Tensor, layout: Layout,
                 slot_buf: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None,
                 use_ws: bool = True) -> torch.Tensor:
    """expert_weights [E][...] (one layer), phy2log int32 [Phi] (one plan), slot_buf [S][...].

    ws: the fill-list workspace (slot_fill_workspace); one is taken from torch's
    allocator when not given, unless use_ws is False (the form without a list)."""
    if not (expert_weights.is_cuda and slot_buf.is_cuda and expert_weights.is_contiguous()
            and slot_buf.is_contiguous()):
        raise EPBalanceError("weights and slot buffer must be contiguous device tensors")
    _arg(phy2log, torch.int32, (layout.num_phys,), "phy2log")
    total = expert_weights.numel() * expert_weights.element_size()
    if total % layout.num_experts != 0:
        raise EPBalanceError("expert_weights must hold the same number of bytes for every expert")
    bpe = total // layout.num_experts
    if slot_buf.numel() * slot_buf.element_size() < layout.num_spare * bpe:
        raise EPBalanceError("slot_buf is smaller than S * bytes_per_expert")
    if ws is None and use_ws:
        ws = slot_fill_workspace(layout, expert_weights.device)
    if ws is not None and not (ws.is_cuda and ws.is_contiguous()):
        raise EPBalanceError("ws must be a contiguous device tensor")
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib().ep_slot_fill(_ptr(expert_weights), bpe, _ptr(phy2log), layout.ref(), _ptr(slot_buf),
                            _ptr(ws), nbytes, _stream(stream))
    _check(rc, "ep_slot_fill")
    return slot_buf


def ep_balance_stats(load: torch.Tensor, phy_quota: torch.Tensor, layout: Layout, stats=None,
                     imbalance=None, rank_load=None, want_rank_load=True, stream=None):
    """-> (stats int64 [P][4], imbalance float64 [P][2], rank_load int32 [P][2][R] or None)."""
    _dev(load, torch.int32, "load")
    P = load.shape[0]
    _arg(load, torch.int32, (P, layout.num_experts), "load")
    _arg(phy_quota, torch.int32, (P, layout.num_phys), "phy_quota")
    dev = load.device
    stats = torch.empty((P, 4), dtype=torch.int64, device=dev) if stats is None else stats
    imbalance = torch.empty((P, 2), dtype=torch.float64, device=dev) if imbalance is None else imbalance
    if rank_load is None and want_rank_load:
        rank_load = torch.empty((P, 2, layout.num_ranks), dtype=torch.int32, device=dev)
    _arg(stats, torch.int64, (P, 4), "stats"); _arg(imbalance, torch.float64, (P, 2), "imbalance")
    if rank_load is not None:
        _arg(rank_load, torch.int32, (P, 2, layout.num_ranks), "rank_load")
    rc = lib().ep_balance_stats(_ptr(load), _ptr(phy_quota), P, layout.ref(), _ptr(stats),
                                _ptr(imbalance), _ptr(rank_load), _stream(stream))
    _check(rc, "ep_balance_stats")
    return stats, imbalance, rank_load


def plan_rows(plan: PlanOut, a: int, b: int) -> PlanOut:
    """Plans a..b-1 of a batch of plan outputs (views, no copy)."""
    return PlanOut(plan.phy2log[a:b], plan.phy_quota[a:b], plan.logcnt[a:b], plan.log2phy[a:b],
                   plan.steps[a:b])


EP_MAX_CHUNKS = 16


class PathPipeline:
    """hist -> plan -> reroute over a batch of plans, cut into chunks of plans and
    overlapped across three streams by the library's ep_route_pipelined: the
    planner of chunk c runs while the histogram of chunk c + 1 streams, and the
    reroute of chunk c while the planner of chunk c + 1 runs.  The outputs are
    those of the same calls made in order on one stream.  Owns the three side
    streams (taken one after another from torch's pool, so that they sit on
    three different hardware queues), the events and the per-chunk workspaces;
    the caller owns inputs and outputs.  run() only enqueues: it is ordered
    after earlier work on the caller's stream, and later work on that stream
    waits for it."""

    def __init__(self, layout: Layout, num_plans: int, pairs_per_plan: int, chunks=2, device=None):
        """chunks: a number of equal chunks, or the list of chunk sizes (plans).
        The planner of a chunk takes about as long as its slowest plan, whatever
        the chunk's size, and the planners run one after another; a first chunk
        of about a third of the plans lets its planner run under the histogram of
        the rest, and the second planner under the first chunk's reroute."""
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        if isinstance(chunks, int):
            n = max(1, min(chunks, int(num_plans)))
            base, extra = divmod(int(num_plans), n)
            sizes = [base + (1 if c < extra else 0) for c in range(n)]
        else:
            sizes = [int(x) for x in chunks]
        if not sizes or min(sizes) < 1 or sum(sizes) != int(num_plans) or len(sizes) > EP_MAX_CHUNKS:
            raise ValueError(f"chunk sizes {sizes} do not split {num_plans} plans (at most {EP_MAX_CHUNKS} chunks)")
        self.bounds = []
        a = 0
        for s in sizes:
            self.bounds.append((a, a + s))
            a += s
        self.layout = layout
        self.num_plans, self.pairs_per_plan = int(num_plans), int(pairs_per_plan)
        self._sizes = (ctypes.c_int32 * len(sizes))(*sizes)
        nbytes = lib().ep_pipeline_workspace_bytes(self.pairs_per_plan, self._sizes, len(sizes), layout.num_experts)
        self.ws = torch.empty(max(16, nbytes), dtype=torch.uint8, device=dev)
        # default-priority side streams; events created (by a first record) up front
        self.s_hist, self.s_plan, self.s_rr = (torch.cuda.Stream(device=dev) for _ in range(3))
        self._side = (ctypes.c_void_p * 3)(self.s_hist.cuda_stream, self.s_plan.cuda_stream,
                                           self.s_rr.cuda_stream)
        self.events = [torch.cuda.Event() for _ in range(2 + 2 * len(sizes))]
        cur = torch.cuda.current_stream(dev)
        for e in self.events:
            e.record(cur)
        self._ev = (ctypes.c_void_p * len(self.events))(*[e.cuda_event for e in self.events])

    def run(self, topk_ids: torch.Tensor, load: torch.Tensor, status: torch.Tensor, plan: PlanOut,
            phys_ids: torch.Tensor, stream=None):
        if tuple(topk_ids.shape) != (self.num_plans, self.pairs_per_plan):
            raise ValueError(f"topk_ids shape {tuple(topk_ids.shape)} != "
                             f"({self.num_plans}, {self.pairs_per_plan})")
        P, N, lay = self.num_plans, self.pairs_per_plan, self.layout
        _dev(topk_ids, torch.int32, "topk_ids")
        _arg(load, torch.int32, (P, lay.num_experts), "load"); _arg(status, torch.int32, (P,), "status")
        _arg(plan.phy2log, torch.int32, (P, lay.num_phys), "phy2log")
        _plan_args(lay, P, plan.phy_quota, plan.log2phy, plan.logcnt)
        _arg(plan.steps, torch.int32, (P,), "steps")
        _arg(phys_ids, torch.int32, (P, N), "phys_ids")
        rc = lib().ep_route_pipelined(_ptr(topk_ids), N, P, lay.ref(), self._sizes, len(self.bounds), _ptr(load),
                                      _ptr(status), _ptr(plan.phy2log), _ptr(plan.phy_quota), _ptr(plan.logcnt),
                                      _ptr(plan.log2phy), _ptr(plan.steps), _ptr(phys_ids), _ptr(self.ws),
                                      self.ws.numel(), _stream(stream), self._side, self._ev)
        _check(rc, "ep_route_pipelined")


def run_path(topk_ids: torch.Tensor, layout: Layout, stream=None):
    """hist -> plan -> reroute -> stats for a batch of plans; returns a dict of device tensors."""
    load, ws, status = ep_load_histogram(topk_ids, layout, stream=stream)
    plan = ep_plan_quota(load, layout, status=status, stream=stream)
    phys = ep_reroute(topk_ids, layout, plan.phy_quota, plan.log2phy, plan.logcnt, ws, stream=stream)
    stats, imb, rank_load = ep_balance_stats(load, plan.phy_quota, layout, stream=stream)
    return dict(load=load, ws=ws, status=status, plan=plan, phys=phys, stats=stats, imbalance=imb,
                rank_load=rank_load)
