"""CPU oracle for real-time MoE expert load balancing -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports it, and the two share no code.

The arithmetic lives in ``ep_oracle.c`` (plain single-threaded C, built with gcc
by :func:`oracle.build.build`); this module only marshals numpy arrays.  The
exact optimum for tiny instances, the slot-count lower bound and the MILP bounds
for full-size plans are in :mod:`oracle.brute`.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

from .build import LIB_PATH, build

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = os.environ.get("EP_ORACLE_LIB") or LIB_PATH
        if path == LIB_PATH and not os.path.exists(LIB_PATH):
            build()
        _lib = ctypes.CDLL(path)
        i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
        i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
        u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        i32 = ctypes.c_int32
        i64 = ctypes.c_int64
        _lib.or_histogram.argtypes = [i32p, i64, i32, i32p, ctypes.POINTER(ctypes.c_int64)]
        _lib.or_histogram.restype = ctypes.c_int
        _lib.or_plan.argtypes = [i32, i32, i32p, i32p, i32p, i32p, i32p, i32p, i32p, i32p, i32,
                                 ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
        _lib.or_plan.restype = ctypes.c_int
        _lib.or_plan_domain.argtypes = [i32, i32, i32p, i32p, i32p, i32p, i32p, i32p, i32p, i32p, i32, i32,
                                        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_int32)]
        _lib.or_plan_domain.restype = ctypes.c_int
        _lib.or_reroute.argtypes = [i32p, i64, i32, i32p, i32p, i32p, i32, i32p]
        _lib.or_reroute.restype = ctypes.c_int64
        _lib.or_slot_fill.argtypes = [u8p, i64, i32, i32, i32p, i32p, i32p, i32p, u8p]
        _lib.or_slot_fill.restype = ctypes.c_int
        _lib.or_stats.argtypes = [i32, i32, i32p, i32p, i32p, i32p, i32p, i64p, i32p, f64p]
        _lib.or_stats.restype = ctypes.c_int
        _lib.or_layout.argtypes = [i32, i32, i32p, i32p, i32p, i32p, i32p, i32p, i32p]
        _lib.or_layout.restype = ctypes.c_int
        _lib.or_waterfill.argtypes = [i64, i32, i64p, i32p, i64p]
        _lib.or_waterfill.restype = ctypes.c_int
        _lib.or_dispatch.argtypes = [i32p, i64, i32, i32, i32p, i32p, i32p, i32, i64p, i32p, i32p]
        _lib.or_dispatch.restype = ctypes.c_int64
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        _lib.or_grad_reduce.argtypes = [f32p, i64, f32p, i32, i32, i32p, i32p, i32p, i32p, i32p, i32]
        _lib.or_grad_reduce.restype = ctypes.c_int
    return _lib


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


@dataclass
class Layout:
    """Native placement + spare slots, as the oracle numbers them."""

    num_experts: int
    num_ranks: int
    native_count: np.ndarray
    native_experts: np.ndarray
    spare_count: np.ndarray

    @classmethod
    def of(cls, E, R, native_count, native_experts, spare_count) -> "Layout":
        return cls(int(E), int(R), _i32(native_count), _i32(native_experts), _i32(spare_count))

    @classmethod
    def from_workload(cls, wl) -> "Layout":
        return cls.of(wl.num_experts, wl.num_ranks, wl.native_count, wl.native_experts(), wl.spare_count)

    @property
    def num_spare(self) -> int:
        return int(self.spare_count.sum())

    @property
    def num_phys(self) -> int:
        return self.num_experts + self.num_spare

    @property
    def max_replicas(self) -> int:
        return min(self.num_ranks, 1 + self.num_spare)

    def args(self):
        return (self.num_experts, self.num_ranks, self.native_count, self.native_experts, self.spare_count)

    def slots(self):
        """(first_slot[R+1], slot_home[Phi], slot_rank[Phi], spare_slot[S])."""
        R, Phi, S = self.num_ranks, self.num_phys, self.num_spare
        first = np.zeros(R + 1, np.int32)
        home = np.zeros(Phi, np.int32)
        rank = np.zeros(Phi, np.int32)
        spare = np.zeros(max(S, 1), np.int32)
        rc = lib().or_layout(*self.args(), first, home, rank, spare)
        if rc != 0:
            raise ValueError(f"oracle: bad layout ({rc})")
        return first, home, rank, spare[:S]


def histogram(ids: np.ndarray, num_experts: int):
    """Per-expert load of one plan and the number of IDs >= E."""
    ids = _i32(ids).reshape(-1)
    load = np.zeros(num_experts, np.int32)
    bad = ctypes.c_int64(0)
    lib().or_histogram(ids, ids.size, num_experts, load, ctypes.byref(bad))
    return load, int(bad.value)


@dataclass
class Plan:
    phy2log: np.ndarray     # [Phi]
    phy_quota: np.ndarray   # [Phi]
    logcnt: np.ndarray      # [E]
    log2phy: np.ndarray     # [E][rho]
    steps: int
    cap_hit: int
    bad_load: int = 0       # a load < 0 or a total above INT32_MAX: no move was made


def plan(load: np.ndarray, layout: Layout, ranks_per_domain: int = 0) -> Plan:
    """ranks_per_domain > 0 keeps every replica in its native rank's domain (rank // D)."""
    E, Phi, rho = layout.num_experts, layout.num_phys, layout.max_replicas
    load = _i32(load).reshape(-1)
    assert load.size == E
    phy2log = np.zeros(Phi, np.int32)
    quota = np.zeros(Phi, np.int32)
    logcnt = np.zeros(E, np.int32)
    log2phy = np.zeros(E * rho, np.int32)
    steps = ctypes.c_int32(0)
    cap = ctypes.c_int32(0)
    bad = ctypes.c_int32(0)
    rc = lib().or_plan_domain(*layout.args(), load, phy2log, quota, logcnt, log2phy, rho,
                              int(ranks_per_domain), ctypes.byref(steps), ctypes.byref(cap), ctypes.byref(bad))
    if rc != 0:
        raise ValueError(f"oracle: bad layout ({rc})")
    return Plan(phy2log, quota, logcnt, log2phy.reshape(E, rho), int(steps.value), int(cap.value),
                int(bad.value))


def reroute(ids: np.ndarray, num_experts: int, phy_quota, log2phy, logcnt):
    """Physical slot of every pair; returns (phys, number of valid pairs left unplaced)."""
    ids = _i32(ids).reshape(-1)
    log2phy = _i32(log2phy)
    rho = log2phy.shape[-1]
    phys = np.zeros(ids.size, np.int32)
    unplaced = lib().or_reroute(ids, ids.size, num_experts, _i32(phy_quota), log2phy.reshape(-1),
                                _i32(logcnt), rho, phys)
    return phys, int(unplaced)


def slot_fill(weights: np.ndarray, phy2log, layout: Layout, slot_buf: np.ndarray) -> np.ndarray:
    """Copy each used spare slot's expert row of ``weights`` into ``slot_buf`` (in place).

    ``weights`` holds E rows and ``slot_buf`` S rows of the same byte size; both
    are C-contiguous numpy arrays of any dtype (bf16 travels as uint16).
    """
    w = np.ascontiguousarray(weights).view(np.uint8).reshape(layout.num_experts, -1)
    W = w.shape[1]
    assert slot_buf.flags["C_CONTIGUOUS"]
    out = slot_buf.view(np.uint8).reshape(-1)
    assert out.size == layout.num_spare * W
    buf = out if out.size else np.zeros(1, np.uint8)
    rc = lib().or_slot_fill(w.reshape(-1), W, *layout.args(), _i32(phy2log), buf)
    if rc != 0:
        raise ValueError(f"oracle: bad layout ({rc})")
    return slot_buf


@dataclass
class Stats:
    max_before: int
    max_after: int
    total: int
    replicas_used: int
    rank_before: np.ndarray
    rank_after: np.ndarray
    imbalance_before: float
    imbalance_after: float

    def as_row(self) -> np.ndarray:
        return np.array([self.max_before, self.max_after, self.total, self.replicas_used], np.int64)


def stats(load, phy_quota, layout: Layout) -> Stats:
    R = layout.num_ranks
    st = np.zeros(4, np.int64)
    rl = np.zeros(2 * R, np.int32)
    imb = np.zeros(2, np.float64)
    rc = lib().or_stats(*layout.args(), _i32(load), _i32(phy_quota), st, rl, imb)
    if rc != 0:
        raise ValueError(f"oracle: bad layout ({rc})")
    return Stats(int(st[0]), int(st[1]), int(st[2]), int(st[3]), rl[:R].copy(), rl[R:].copy(),
                 float(imb[0]), float(imb[1]))


def waterfill(T: int, backgrounds, ranks) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(backgrounds, np.int64))
    r = _i32(ranks)
    q = np.zeros(b.size, np.int64)
    lib().or_waterfill(int(T), b.size, b, r, q)
    return q


def dispatch(ids: np.ndarray, num_experts: int, phy_quota, log2phy, logcnt):
    """Dispatch layout of one plan: (slot_off[Phi+1], pos[N], src[N], placed pairs)."""
    ids = _i32(ids).reshape(-1)
    log2phy = _i32(log2phy)
    rho = log2phy.shape[-1]
    q = _i32(phy_quota)
    off = np.zeros(q.size + 1, np.int64)
    pos = np.zeros(max(ids.size, 1), np.int32)
    src = np.zeros(max(ids.size, 1), np.int32)
    placed = lib().or_dispatch(ids, ids.size, num_experts, q.size, q, log2phy.reshape(-1), _i32(logcnt),
                               rho, off, pos, src)
    return off, pos[: ids.size], src[: ids.size], int(placed)


def grad_reduce(native_grads: np.ndarray, slot_grads: np.ndarray, layout: Layout, log2phy, logcnt):
    """In place: every replicated expert's row of native_grads becomes the fp32
    fold of its instances' rows in ascending slot order."""
    assert native_grads.dtype == np.float32 and native_grads.flags["C_CONTIGUOUS"]
    n = native_grads.shape[1]
    sg = np.ascontiguousarray(slot_grads, dtype=np.float32).reshape(-1)
    l2p = _i32(log2phy)
    rc = lib().or_grad_reduce(native_grads.reshape(-1), n, sg if sg.size else np.zeros(1, np.float32),
                              *layout.args(), l2p.reshape(-1), _i32(logcnt), l2p.shape[-1])
    if rc != 0:
        raise ValueError(f"oracle: bad layout ({rc})")
    return native_grads


def run_path(ids_2d: np.ndarray, layout: Layout):
    """All five steps for a batch of plans; returns dict of stacked outputs."""
    P = ids_2d.shape[0]
    E = layout.num_experts
    loads, bads, plans, phys, sts = [], [], [], [], []
    for p in range(P):
        ld, bad = histogram(ids_2d[p], E)
        pl = plan(ld, layout)
        ph, unplaced = reroute(ids_2d[p], E, pl.phy_quota, pl.log2phy, pl.logcnt)
        assert unplaced == 0
        loads.append(ld); bads.append(bad); plans.append(pl); phys.append(ph)
        sts.append(stats(ld, pl.phy_quota, layout))
    return dict(load=np.stack(loads), bad=np.array(bads), plans=plans, phys=np.stack(phys), stats=sts)
