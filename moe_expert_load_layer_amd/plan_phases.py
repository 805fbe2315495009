"""Per-phase cycle split of the rank-per-lane planner, one plan per launch.

Needs the profiling build (the normal library compiles the phase marks out):

    python -m moe_expert_load_layer_amd.build --plan-phases      # libepbalance_phases.so
    python -m moe_expert_load_layer_amd.plan_phases [workload ...]

For plans 0..3 of each workload it times one single-plan launch with HIP events
on the normal library and on the profiling build, checks that both plan
identically, and prints the cycles per committed move of each phase (s_memtime
stamps of lane 0; the marks themselves add about 40 cycles each).
"""
from __future__ import annotations

import ctypes
import os
import statistics
import sys

import torch

import moe_expert_load_layer_amd as ep
from .build import PHASES_LIB_PATH

PHASES = ("hottest rank", "candidate read-out", "candidate pick", "instances and destination",
          "ranking", "m*, division, new load", "commit", "loop")


def _use(path: str) -> ctypes.CDLL:
    ep._lib = None
    ep.LIB_PATH = path
    return ep.lib()


def _timed(fn, stream, reps: int = 10) -> float:
    for _ in range(2):
        fn()
    xs = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream); fn(); b.record(stream)
        xs.append((a, b))
    torch.cuda.synchronize()
    return statistics.median([a.elapsed_time(b) for a, b in xs]) * 1e3


def main(names) -> int:
    import workloads as W
    if not os.path.exists(PHASES_LIB_PATH):
        print(f"{PHASES_LIB_PATH} is not built: python -m moe_expert_load_layer_amd.build --plan-phases",
              file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    normal = ep.LIB_PATH
    print("| workload | plan | moves | tries | ranking iterations | launch µs (normal / profiling build) | "
          + " | ".join(PHASES) + " | cycles per move |")
    print("|---|---|---|---|---|---|" + "---|" * len(PHASES) + "---|")
    for name in names:
        wl = W.get(name)
        _use(normal)
        ids = W.make_ids(wl, device=dev, plans=[0, 1, 2, 3])
        lay = ep.Layout.from_workload(wl, device=dev)
        load, _, _ = ep.ep_load_histogram(ids, lay)
        del ids
        for p in range(4):
            ld = load[p:p + 1].contiguous()
            ref = ep.alloc_plan(1, lay, dev)
            _use(normal)
            t_normal = _timed(lambda: ep.ep_plan_quota(ld, lay, out=ref), stream)
            out = ep.alloc_plan(1, lay, dev)
            L = _use(PHASES_LIB_PATH)
            t_prof = _timed(lambda: ep.ep_plan_quota(ld, lay, out=out), stream)
            torch.cuda.synchronize()
            for f in ("phy2log", "phy_quota", "logcnt", "log2phy", "steps"):
                if not torch.equal(getattr(out, f), getattr(ref, f)):
                    raise SystemExit(f"{name} plan {p}: the profiling build planned differently ({f})")
            buf = (ctypes.c_ulonglong * 16)()
            L.ep_plan_phases_read.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.c_int]
            if L.ep_plan_phases_read(buf, 1) != 0:
                raise SystemExit("ep_plan_phases_read failed")
            moves = max(int(buf[10]), 1)
            cells = " | ".join(f"{buf[k] / moves:.0f}" for k in range(8))
            print(f"| {name} | {p} | {buf[10]} | {buf[8]} | {buf[9]} | {t_normal:.1f} / {t_prof:.1f} | {cells} | "
                  f"{buf[11] / moves:.0f} |", flush=True)
        _use(normal)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:] or ["qwen3_235b", "deepseek_v3", "glm_4_5", "stress"]))
