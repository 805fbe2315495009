"""Benchmark of the real-time expert load-balancing path on one MI355X.

One step = the whole path over one microbatch of the Qwen3-235B-like workload
(128 experts, top-8, EP64 with 2 native + 1 spare slot per rank, 8192 tokens
per rank, 94 MoE layers):
  ep_load_histogram (94 plans) -> ep_plan_quota (94) -> ep_reroute (94)
  -> ep_balance_stats (94) -> ep_slot_fill once per layer (94 launches into the
  one cross-layer slot buffer, 3x4096x1536 bf16 per expert).
The first three run as --chunks chunks of plans overlapped across three streams
(the planner of one chunk under the histogram or reroute of another); the same
path as three launches on one stream is timed beside it.
Inputs are synthetic, seeded, and resident in HBM before timing starts.

value = (token,k) pairs per second through hist + plan + reroute (HIP events
around that phase in every timed step); ms_per_step is the whole step
including the slot fills and statistics.  The `kernels` object also carries
single-layer latencies: each kernel alone, and the whole chain of one layer in
one call on one stream (`route_chain_us_single_layer`), the latency a forward
pass that plans layer by layer sees.

Byte rules (algorithmic bytes per unit of work):
  path        12 B per pair: the ID read by the histogram (4), read again and the
              physical slot written by the reroute (4 + 4)
  histogram   4 B per pair; reroute 8 B per pair (the same split)
  slot fill   2 x bytes_per_expert per filled spare slot (each slot's expert
              read and the slot written)
Beside each, the bytes the kernels actually move: with E <= 256 the histogram
writes a one-byte copy of each ID that the reroute reads instead (5 + 5 B per
pair with the count rows), and the slot fill reads each distinct expert once for
all the slots that hold it ((distinct experts + filled slots) x bytes_per_expert).

The roofline object covers the dominant kernel, the slot fill: `achieved` and
`frac` on the first rule (which can pass 1.0: the fill reads a replicated expert
once for up to four of its slots, so it moves fewer bytes than that rule counts),
`achieved_moved` and `frac_moved` on the bytes moved,
from the mean launch time measured with HIP events on the stream the fills run
on.  `traffic` is the HBM bytes per launch from the rocprofv3 FETCH_SIZE and
WRITE_SIZE summary committed for this kernel source (null when the source has
changed since).  The `workloads` object repeats the measurement, compactly, for
every workload, with the dispatch layout over all plans beside it.  The CPU baseline times the C oracle on a bounded sample of the
same layers on the host (hist + plan + reroute, and the slot fill as memcpy).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_expert_load_layer_amd as ep  # noqa: E402
import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "(token,k) pairs/s via hist+plan+reroute; plan µs/layer at EP64; HBM GB/s"

PATH_BYTES_PER_PAIR = 12.0      # hist 4 (ID in) + reroute 8 (ID in, slot out)
HIST_BYTES_PER_PAIR = 4.0
REROUTE_BYTES_PER_PAIR = 8.0
FILL_RULE = "2 x bytes_per_expert per filled spare slot (read + write per slot)"
FILL_MOVED_RULE = "(distinct experts in filled spare slots + filled slots) x bytes_per_expert"


def profile_traffic(workload: str):
    """HBM bytes per slot-fill launch from the committed rocprofv3 summary of this
    workload (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by the plain-copy
    calibration it records), or None when the summary was taken on another
    version of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"slot_fill_{workload}.md")
    if not os.path.exists(path):
        return None, None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("traffic-record:"):
                for kv in line.split(":", 1)[1].split():
                    k, v = kv.split("=", 1)
                    fields[k] = v
    if not fields or fields.get("kernel_sha") != _src_sha("slotfill.hip"):
        return None, os.path.relpath(path, ROOT)
    kib = 1024.0
    b = (float(fields["fetch_kib"]) * float(fields["fetch_scale"]) +
         float(fields["write_kib"]) * float(fields["write_scale"])) * kib
    return b, os.path.relpath(path, ROOT)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _src_sha(name: str) -> str:
    with open(os.path.join(ROOT, "moe_expert_load_layer_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _elapsed(pairs):
    return [a.elapsed_time(b) for a, b in pairs]


def cpu_baseline(ids_host: np.ndarray, wl, budget_s: float):
    """The oracle on the host over as many leading layers as fit the time budget."""
    import oracle

    lay = oracle.Layout.from_workload(wl)
    E = wl.num_experts
    done, pairs, t_used = 0, 0, 0.0
    outs = []
    for p in range(ids_host.shape[0]):
        t0 = time.perf_counter()
        ld, _ = oracle.histogram(ids_host[p], E)
        pl = oracle.plan(ld, lay)
        ph, _ = oracle.reroute(ids_host[p], E, pl.phy_quota, pl.log2phy, pl.logcnt)
        t_used += time.perf_counter() - t0
        outs.append((ld, pl, ph))
        done += 1
        pairs += ids_host.shape[1]
        if t_used >= budget_s:
            break
    return dict(value=pairs / t_used, unit="pairs/s", cores=1, kind="oracle",
                sample=f"hist+plan+reroute of the first {done} of {ids_host.shape[0]} layers "
                       f"({pairs} pairs), single host thread, {t_used:.1f} s"), outs


def spare_slots(wl):
    """Physical slot of every spare ordinal (rank-major; natives first in a rank)."""
    out, s0 = [], 0
    for nc_r, sc_r in zip(wl.native_count, wl.spare_count):
        s0 += int(nc_r)
        out.extend(range(s0, s0 + int(sc_r)))
        s0 += int(sc_r)
    return out


def fill_rates(wl, phy2log_host: np.ndarray, fill_ms: np.ndarray):
    """Slot-fill rates for the layers whose mean launch times are fill_ms, on the
    per-slot rule (2 x W per filled slot) and on the bytes moved ((distinct
    experts + filled slots) x W)."""
    bpe = wl.bytes_per_expert
    sp = phy2log_host[: len(fill_ms)][:, spare_slots(wl)]
    filled = (sp >= 0).sum(axis=1).astype(np.float64)
    distinct = np.array([len(np.unique(r[r >= 0])) for r in sp], np.float64)
    t = float(np.mean(fill_ms)) * 1e-3
    b = float((2 * bpe * filled).mean())
    mb = float((bpe * (distinct + filled)).mean())
    return {"ms": float(np.mean(fill_ms)), "bytes": b, "GBps": b / t / 1e9, "frac": b / t / 1e9 / HBM_PEAK_GBPS,
            "moved_bytes": mb, "moved_GBps": mb / t / 1e9, "moved_frac": mb / t / 1e9 / HBM_PEAK_GBPS,
            "filled": float(filled.mean()), "distinct": float(distinct.mean())}


def moved_bytes_per_pair(N: int, P: int, E: int):
    """Bytes per pair the histogram and the reroute move: with E <= 256 the
    histogram writes a one-byte copy of each ID that the reroute reads instead
    of the int32 ID (4 in + 1 out, 1 in + 4 out); otherwise 4 in, and 4 + 4.
    Both also carry the count rows: one row of E + 1 int32 per sub-block,
    written by the histogram and read by the reroute."""
    h, r = (5.0, 5.0) if E <= 256 else (4.0, 8.0)
    sub = ep.ep_sub_block_pairs(N, P, E)
    rows = -(-N // sub) * (E + 1) * 4 / N if N else 0.0
    return h + rows, r + rows


def kernel_rates(pairs, hist_ms, rr_ms, serial_ms, plan_ms, path_ms, hist_moved, rr_moved):
    g = lambda bpp, ms: bpp * pairs / (ms * 1e-3) / 1e9      # GB/s
    return {
        "path_GBps": g(PATH_BYTES_PER_PAIR, path_ms),
        "path_frac": g(PATH_BYTES_PER_PAIR, path_ms) / HBM_PEAK_GBPS,
        "path_stream_frac": g(PATH_BYTES_PER_PAIR, hist_ms + rr_ms) / HBM_PEAK_GBPS,
        "path_serial_frac": g(PATH_BYTES_PER_PAIR, serial_ms) / HBM_PEAK_GBPS,
        "per_kernel": {
            "hist_ms": hist_ms, "reroute_ms": rr_ms, "plan_ms": plan_ms,
            "hist_rule_bytes_per_pair": HIST_BYTES_PER_PAIR,
            "hist_rule_frac": g(HIST_BYTES_PER_PAIR, hist_ms) / HBM_PEAK_GBPS,
            "reroute_rule_bytes_per_pair": REROUTE_BYTES_PER_PAIR,
            "reroute_rule_frac": g(REROUTE_BYTES_PER_PAIR, rr_ms) / HBM_PEAK_GBPS,
            "hist_moved_bytes_per_pair": hist_moved,
            "hist_moved_GBps": g(hist_moved, hist_ms), "hist_moved_frac": g(hist_moved, hist_ms) / HBM_PEAK_GBPS,
            "reroute_moved_bytes_per_pair": rr_moved,
            "reroute_moved_GBps": g(rr_moved, rr_ms),
            "reroute_moved_frac": g(rr_moved, rr_ms) / HBM_PEAK_GBPS,
        },
    }


def cpu_slot_fill(weights: torch.Tensor, phy2log_host: np.ndarray, wl, budget_s: float):
    """The oracle's slot fill (a memcpy per filled spare slot) on the host over a
    host copy of one layer's weights, for as many layers as fit the budget."""
    import oracle

    lay = oracle.Layout.from_workload(wl)
    w = weights.cpu().view(torch.int16).numpy()
    buf = np.empty((wl.num_spare, w.shape[1]), np.int16)
    done, nbytes, t_used = 0, 0.0, 0.0
    spare = spare_slots(wl)
    for p in range(phy2log_host.shape[0]):
        t0 = time.perf_counter()
        oracle.slot_fill(w, phy2log_host[p], lay, buf)
        t_used += time.perf_counter() - t0
        nbytes += 2.0 * wl.bytes_per_expert * int((phy2log_host[p][spare] >= 0).sum())
        done += 1
        if t_used >= budget_s:
            break
    return {"value": nbytes / t_used, "unit": "B/s", "bytes_rule": FILL_RULE, "cores": 1, "kind": "oracle",
            "sample": f"slot fill (memcpy per filled slot) of the first {done} of {phy2log_host.shape[0]} "
                      f"layers over a host copy of one layer's weights, single host thread, {t_used:.1f} s"}


def workload_summary(name: str, dev, cpu_bound: bool, fill_layers: int = 16):
    """Compact numbers for one workload at full size: the path (fastest of one
    stream and two chunks), each kernel alone, single-layer latencies, the
    dispatch layout over all plans, the slot fill over its first layers, and the
    balance."""
    wl = W.get(name)
    P, N, E, S = wl.num_plans, wl.pairs_per_plan, wl.num_experts, wl.num_spare
    ids = W.make_ids(wl, device=dev)
    weights = W.make_weights(wl, device=dev)
    lay = ep.Layout.from_workload(wl, device=dev)
    slot = torch.empty((max(S, 1), weights.shape[1]), dtype=weights.dtype, device=dev)
    fws = ep.slot_fill_workspace(lay, dev)
    load = torch.empty((P, E), dtype=torch.int32, device=dev)
    ws = ep.workspace(ids, lay)
    status = torch.empty(P, dtype=torch.int32, device=dev)
    plan = ep.alloc_plan(P, lay, dev)
    phys = torch.empty_like(ids)
    stream = torch.cuda.current_stream()

    def timed(fn, reps=5):
        fn()
        xs = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
            a.record(stream); fn(); b.record(stream)
            xs.append((a, b))
        torch.cuda.synchronize()
        return statistics.median(_elapsed(xs))

    def serial():
        ep.ep_load_histogram(ids, lay, load=load, ws=ws, status=status)
        ep.ep_plan_quota(load, lay, out=plan, status=status)
        ep.ep_reroute(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws, phys_ids=phys)

    t_serial = timed(serial)
    best, best_chunks = t_serial, [P]
    for first in sorted({round(0.37 * P), P // 2}):
        if 1 <= first < P:
            for _ in range(2):  # two pipelines: each has streams of its own (see main)
                pp = ep.PathPipeline(lay, P, N, chunks=[first, P - first], device=dev)
                t = timed(lambda: pp.run(ids, load, status, plan, phys))
                if t < best * 0.98:
                    best, best_chunks = t, [first, P - first]
                del pp
    t_hist = timed(lambda: ep.ep_load_histogram(ids, lay, load=load, ws=ws, status=status))
    t_plan = timed(lambda: ep.ep_plan_quota(load, lay, out=plan, status=status))
    t_rr = timed(lambda: ep.ep_reroute(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws, phys_ids=phys))
    serial()
    soff = torch.empty((P, lay.num_phys + 1), dtype=torch.int32, device=dev)
    dpos = torch.empty_like(ids)
    dsrc = torch.empty_like(ids)
    t_disp = timed(lambda: ep.ep_dispatch_layout(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws,
                                                 slot_offsets=soff, dispatch_pos=dpos, dispatch_src=dsrc), reps=3)
    del soff, dpos, dsrc
    ids1, load1 = ids[:1], load[:1].clone()
    pl1 = ep.alloc_plan(1, lay, dev)
    t_plan1 = timed(lambda: ep.ep_plan_quota(load1, lay, out=pl1), reps=15) * 1e3
    hm, rm = moved_bytes_per_pair(N, P, E)
    kern = kernel_rates(P * N, t_hist, t_rr, t_serial, t_plan, best, hm, rm)

    nf = min(P, fill_layers)
    fms = []
    if S > 0:
        for _ in range(2):
            ep.ep_slot_fill(weights, plan.phy2log[0], lay, slot, ws=fws)
        ev = []
        for rep in range(2):
            for l in range(nf):
                a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
                a.record(stream); ep.ep_slot_fill(weights, plan.phy2log[l], lay, slot, ws=fws); b.record(stream)
                ev.append((a, b))
        torch.cuda.synchronize()
        fms = np.array(_elapsed(ev)).reshape(2, nf).mean(axis=0)
    fill = fill_rates(wl, plan.phy2log.cpu().numpy(), fms) if S > 0 else None

    stats, imb, _ = ep.ep_balance_stats(load, plan.phy_quota, lay, want_rank_load=False)
    imb_np = imb.cpu().numpy()
    out = {
        "path_pairs_per_s": P * N / (best * 1e-3), "path_ms": best, "path_chunks": best_chunks,
        "path_one_stream_ms": t_serial,
        "path_12B_frac": kern["path_frac"], "path_12B_frac_streaming_kernels": kern["path_stream_frac"],
        "hist_ms": t_hist, "reroute_ms": t_rr,
        "hist_rule_frac": kern["per_kernel"]["hist_rule_frac"],
        "reroute_rule_frac": kern["per_kernel"]["reroute_rule_frac"],
        "hist_moved_frac": kern["per_kernel"]["hist_moved_frac"],
        "reroute_moved_frac": kern["per_kernel"]["reroute_moved_frac"],
        "plan_us_per_layer_batched": t_plan * 1e3 / P, "plan_us_single_layer": t_plan1,
        "dispatch_layout_ms": t_disp,
        "dispatch_layout_12B_frac": 12.0 * P * N / (t_disp * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "imbalance_before_mean": float(imb_np[:, 0].mean()),
        "imbalance_after_mean": float(imb_np[:, 1].mean()),
        "imbalance_after_max": float(imb_np[:, 1].max()),
        "status_nonzero": int((status != 0).sum().item()),
        "planner_steps_max": int(plan.steps.max().item()),
    }
    if fill is not None:
        out.update({"fill_ms_per_layer": fill["ms"], "fill_frac": fill["frac"],
                    "fill_moved_frac": fill["moved_frac"], "fill_layers": nf,
                    "filled_slots_mean": fill["filled"], "distinct_experts_mean": fill["distinct"]})
    if cpu_bound:
        # CPU side: the slot-count lower bound on the max rank load of every
        # layer (no plan beats it), as an imbalance beside the planner's
        from oracle.brute import slot_lower_bound
        ld = load.cpu().numpy()
        lbs = []
        for p in range(P):
            tot = int(ld[p].sum())
            if tot > 0:
                lbs.append((slot_lower_bound(ld[p], wl.num_ranks, S) * wl.num_ranks / tot, float(imb_np[p, 1])))
        if lbs:
            lb = np.array(lbs)
            out["imbalance_lower_bound_mean"] = float(lb[:, 0].mean())
            out["imbalance_after_over_bound_max"] = float((lb[:, 1] / lb[:, 0]).max())
    del ids, weights, slot, ws, phys, load, plan
    torch.cuda.empty_cache()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen3_235b")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work (0 = skip)")
    ap.add_argument("--latency-reps", type=int, default=30)
    ap.add_argument("--chunks", default="auto",
                    help="plans per step cut into chunks overlapped across streams: 'auto' (the "
                         "fastest of one stream and a first chunk of 25/37/50%% of the plans, timed "
                         "during warmup), a number of equal chunks (1 = one stream), or "
                         "comma-separated sizes")
    ap.add_argument("--workloads", default="all",
                    help="after the headline: a compact measurement of the other workloads ('all', "
                         "'none' or a comma-separated list of names)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "path (all-gather of per-rank histograms, xGMI slot fill) is not built.", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # one elementwise kernel that reads and writes 1 GiB each (a plain copy
        # with a sign flip; torch's own contiguous copy is a DMA, not a kernel)
        n = 1 << 28
        src = torch.empty(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))
        return 0
    wl = W.get(args.workload)
    P, N, E, S = wl.num_plans, wl.pairs_per_plan, wl.num_experts, wl.num_spare
    bpe = wl.bytes_per_expert
    print(f"[bench] workload {wl.name}: P={P} N={N} E={E} R={wl.num_ranks} S={S} "
          f"bytes/expert={bpe}", file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    ids = W.make_ids(wl, device=dev)
    weights = W.make_weights(wl, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    lay = ep.Layout.from_workload(wl, device=dev)
    slot = torch.empty((S, weights.shape[1]), dtype=weights.dtype, device=dev)
    fws = ep.slot_fill_workspace(lay, dev)
    load = torch.empty((P, E), dtype=torch.int32, device=dev)
    ws = ep.workspace(ids, lay)
    status = torch.empty(P, dtype=torch.int32, device=dev)
    plan = ep.alloc_plan(P, lay, dev)
    phys = torch.empty_like(ids)
    stats = torch.empty((P, 4), dtype=torch.int64, device=dev)
    imb = torch.empty((P, 2), dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream()

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def run_chunks(c):
        return ep.PathPipeline(lay, P, N, chunks=c, device=dev) if c != 1 else None

    def path_once(pp):
        if pp is None:
            ep.ep_load_histogram(ids, lay, load=load, ws=ws, status=status)
            ep.ep_plan_quota(load, lay, out=plan, status=status)
            ep.ep_reroute(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws, phys_ids=phys)
        else:
            pp.run(ids, load, status, plan, phys)

    tuning = None
    if args.chunks == "auto":
        # A planner launch takes about as long as its slowest plan; overlapping
        # it with another chunk's streaming kernels pays only when that chunk
        # streams for at least as long.  Pick among one stream and a first
        # chunk of 25 / 37 / 50 % of the plans by timing each on this workload
        # (part of the warmup, outside the timed steps).
        cands = [1] + sorted({(f, P - f) for f in (round(0.25 * P), round(0.37 * P), round(0.5 * P))
                              if 1 <= f < P})
        tuning = {}
        best, best_ms, best_pp = 1, None, None
        for c in cands:
            cc = list(c) if c != 1 else 1
            pp = run_chunks(cc)
            path_once(pp)
            xs = []
            for _ in range(5):
                a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
                a.record(stream); path_once(pp); b.record(stream)
                xs.append((a, b))
            torch.cuda.synchronize()
            t_ms = statistics.median(_elapsed(xs))
            tuning["one stream" if cc == 1 else ",".join(map(str, cc))] = t_ms
            # overlap must win clearly: its gain is small where it exists and
            # single timings vary by a few per cent
            if best_ms is None or t_ms < best_ms * (0.98 if best == 1 else 1.0):
                best, best_ms, best_pp = cc, t_ms, pp
        chunks = best
        if best != 1:
            # two kernels overlap only when their streams sit on different
            # hardware queues, and which queue a new stream gets is up to the
            # runtime: time two more pipelines of the chosen chunks (each with
            # streams of its own) and keep the fastest
            for _ in range(2):
                pp = run_chunks(best)
                path_once(pp)
                xs = []
                for _ in range(5):
                    a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
                    a.record(stream); path_once(pp); b.record(stream)
                    xs.append((a, b))
                torch.cuda.synchronize()
                t_ms = statistics.median(_elapsed(xs))
                if t_ms < best_ms:
                    best_ms, best_pp = t_ms, pp
        # the timed steps use the pipeline (and its streams) that was timed here
    elif "," in args.chunks:
        chunks = [int(x) for x in args.chunks.split(",")]
    else:
        chunks = int(args.chunks)
    pipe = best_pp if tuning is not None else run_chunks(chunks)
    rec = dict(path=[], stats=[], fill=[])

    def step(record: bool):
        # events only at the ends of the path: an event between two kernels
        # leaves the GPU idle for a few microseconds
        a = ev()
        path_once(pipe)
        d = ev()
        ep.ep_balance_stats(load, plan.phy_quota, lay, stats=stats, imbalance=imb, want_rank_load=False)
        f = ev()
        fills = []
        for l in range(P):
            x = ev()
            ep.ep_slot_fill(weights, plan.phy2log[l], lay, slot, ws=fws)
            fills.append((x, ev()))
        if record:
            rec["path"].append((a, d)); rec["stats"].append((d, f)); rec["fill"].extend(fills)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    print(f"[bench] {args.steps} timed steps, {wall_ms:.2f} ms/step", file=sys.stderr, flush=True)

    ms = {k: _elapsed(v) for k, v in rec.items()}
    path_ms = statistics.mean(ms["path"])
    pairs_per_s = P * N / (path_ms * 1e-3)

    st = stats.cpu().numpy()
    used = st[:, 3]
    fill_ms = np.array(ms["fill"]).reshape(args.steps, P).mean(axis=0)
    fill = fill_rates(wl, plan.phy2log.cpu().numpy(), fill_ms)
    imb_np = imb.cpu().numpy()

    # single-plan latencies (one layer, as a real forward pass sees them)
    def lat(fn, reps):
        xs = []
        for _ in range(3):
            fn()
        for _ in range(reps):
            a = ev(); fn(); b = ev()
            xs.append((a, b))
        torch.cuda.synchronize()
        return statistics.median(_elapsed(xs)) * 1e3   # us

    # throughput of back-to-back calls: events around `per` calls, median of
    # `reps` such runs, per call (the launch gaps of a lone call do not count)
    def run_ms(fn, reps, per=4):
        xs = []
        for _ in range(2):
            fn()
        for _ in range(reps):
            a = ev()
            for _ in range(per):
                fn()
            b = ev()
            xs.append((a, b))
        torch.cuda.synchronize()
        return statistics.median(_elapsed(xs)) / per

    # the path's phases one at a time, all plans per launch
    ph_hist = run_ms(lambda: ep.ep_load_histogram(ids, lay, load=load, ws=ws, status=status), 5)
    ph_plan = run_ms(lambda: ep.ep_plan_quota(load, lay, out=plan, status=status), 5)
    ph_rr = run_ms(lambda: ep.ep_reroute(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws,
                                         phys_ids=phys), 5)
    # the same path as one stream of three launches, for comparison
    def serial():
        ep.ep_load_histogram(ids, lay, load=load, ws=ws, status=status)
        ep.ep_plan_quota(load, lay, out=plan, status=status)
        ep.ep_reroute(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws, phys_ids=phys)
    ph_serial = run_ms(serial, 5)
    hist_moved, rr_moved = moved_bytes_per_pair(N, P, E)
    kern = kernel_rates(P * N, ph_hist, ph_rr, ph_serial, ph_plan, path_ms, hist_moved, rr_moved)

    ids1 = ids[:1]
    load1 = load[:1].clone()
    ws1 = ep.workspace(ids1, lay)
    st1 = torch.empty(1, dtype=torch.int32, device=dev)
    pl1 = ep.alloc_plan(1, lay, dev)
    ph1 = torch.empty_like(ids1)
    lat_hist = lat(lambda: ep.ep_load_histogram(ids1, lay, load=load1, ws=ws1, status=st1), args.latency_reps)
    lat_plan = lat(lambda: ep.ep_plan_quota(load1, lay, out=pl1), args.latency_reps)
    lat_rr = lat(lambda: ep.ep_reroute(ids1, lay, pl1.phy_quota, pl1.log2phy, pl1.logcnt, ws1, phys_ids=ph1),
                 args.latency_reps)
    # the whole chain for one layer in one call on one stream, as a forward pass
    # without batching runs it (histogram, scan, planner, reroute and the gaps
    # between their launches)
    ld1c, st1c, pl1c, ph1c = load1.clone(), st1.clone(), ep.alloc_plan(1, lay, dev), torch.empty_like(ids1)
    lat_chain = lat(lambda: ep.ep_route_noalloc(ids1, lay, ld1c, st1c, pl1c, ph1c), args.latency_reps)

    # next rows beyond the timed step, one launch over all plans each
    slot_off = torch.empty((P, lay.num_phys + 1), dtype=torch.int32, device=dev)
    dpos = torch.empty_like(ids)
    dsrc = torch.empty_like(ids)
    disp_ms = lat(lambda: ep.ep_dispatch_layout(ids, lay, plan.phy_quota, plan.log2phy, plan.logcnt, ws,
                                                slot_offsets=slot_off, dispatch_pos=dpos,
                                                dispatch_src=dsrc), 5) * 1e-3
    next_rows = {"dispatch_layout_ms": disp_ms,
                 "dispatch_layout_GBps": 12.0 * P * N / (disp_ms * 1e-3) / 1e9}
    # backward: fold replica gradients (fp32, one expert's element count) into the
    # native rows for layer 0's plan
    n_el = bpe // 2
    g_native = torch.zeros((E, n_el), dtype=torch.float32, device=dev)
    g_slot = torch.zeros((S, n_el), dtype=torch.float32, device=dev)
    l2p0, lc0 = plan.log2phy[0].contiguous(), plan.logcnt[0].contiguous()
    red_ms = lat(lambda: ep.ep_replica_grad_reduce(g_native, g_slot, l2p0, lc0, lay), 5) * 1e-3
    lc_h = lc0.cpu().numpy()
    red_bytes = float(((lc_h + 1) * (lc_h >= 2)).sum()) * n_el * 4
    next_rows.update({"grad_reduce_ms": red_ms, "grad_reduce_bytes": red_bytes,
                      "grad_reduce_GBps": red_bytes / (red_ms * 1e-3) / 1e9})
    del g_native, g_slot
    # domain-constrained planner: replicas stay inside 8-rank scale-up domains
    # (one xGMI node); the same loads, all plans in one launch
    lay_d = lay.with_domain(8)
    pl_d = ep.alloc_plan(P, lay_d, dev)
    dom_ms = lat(lambda: ep.ep_plan_quota(load, lay_d, out=pl_d), 5) * 1e-3
    st_d = torch.empty((P, 4), dtype=torch.int64, device=dev)
    imb_d = torch.empty((P, 2), dtype=torch.float64, device=dev)
    ep.ep_balance_stats(load, pl_d.phy_quota, lay_d, stats=st_d, imbalance=imb_d, want_rank_load=False)
    imb_d_np = imb_d.cpu().numpy()
    next_rows.update({"domain_plan_ranks_per_domain": 8,
                      "domain_plan_us_per_layer_batched": dom_ms * 1e3 / P,
                      "domain_imbalance_after_mean": float(imb_d_np[:, 1].mean()),
                      "domain_imbalance_after_max": float(imb_d_np[:, 1].max())})

    traffic, traffic_src = profile_traffic(wl.name)

    out = {
        "metric": METRIC,
        "value": pairs_per_s,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic (seeded Dirichlet(0.3) top-8 routing, bf16 N(0,1) expert weights)",
        "config": {"workload": f"{wl.name}: E={E} top-{wl.top_k} EP{wl.num_ranks} "
                               f"{wl.tokens_per_rank} tokens/rank, {P} layers, {S} spare slots, "
                               f"expert {'x'.join(map(str, wl.expert_shape))} bf16",
                   "pairs_per_step": P * N, "plans_per_step": P},
        # the events bracket one ep_slot_fill call: the one-workgroup list
        # kernel (about 1 % of it) and the copy kernel
        "roofline": {"bound": "hbm", "kernel": "ep_slot_fill (fill_list_kernel + fill_copy_kernel)",
                     "achieved": fill["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": fill["frac"], "traffic": traffic,
                     "bytes_rule": FILL_RULE, "bytes_per_launch": fill["bytes"],
                     "achieved_moved": fill["moved_GBps"], "frac_moved": fill["moved_frac"],
                     "moved_bytes_rule": FILL_MOVED_RULE, "moved_bytes_per_launch": fill["moved_bytes"],
                     "traffic_source": traffic_src,
                     "filled_slots_mean": fill["filled"], "distinct_experts_mean": fill["distinct"],
                     "launch_ms": fill["ms"]},
        "path": {"bytes_per_pair": PATH_BYTES_PER_PAIR,
                 "overlapped_ms": path_ms, "overlapped_GBps": kern["path_GBps"],
                 "overlapped_frac": kern["path_frac"],
                 "streaming_kernels_ms": ph_hist + ph_rr, "streaming_kernels_frac": kern["path_stream_frac"],
                 "one_stream_ms": ph_serial, "one_stream_frac": kern["path_serial_frac"]},
        "phases_ms_per_step": {"path": path_ms, "stats": statistics.mean(ms["stats"]),
                               "fill": float(fill_ms.sum())},
        "phases_ms_alone": {"hist": ph_hist, "plan": ph_plan, "reroute": ph_rr,
                            "path_one_stream": ph_serial},
        "path_chunks": [b - a for a, b in pipe.bounds] if pipe is not None else [P],
        "path_chunk_tuning_ms": tuning,
        "kernels": {**kern["per_kernel"],
                    "plan_us_per_layer_batched": ph_plan * 1e3 / P,
                    "plan_us_single_layer": lat_plan,
                    "hist_us_single_layer": lat_hist,
                    "reroute_us_single_layer": lat_rr,
                    "route_chain_us_single_layer": lat_chain},
        "next_rows": next_rows,
        "balance": {
            "imbalance_before_mean": float(imb_np[:, 0].mean()),
            "imbalance_after_mean": float(imb_np[:, 1].mean()),
            "imbalance_after_max": float(imb_np[:, 1].max()),
            "replicas_used_mean": float(used.mean()),
            "planner_steps_max": int(plan.steps.max().item()),
            "status_nonzero": int((status != 0).sum().item()),
        },
    }
    if wl.microbatches > 1:
        # History-based placement for comparison: each plan uses the replicas
        # planned for the same layer of the previous microbatch, and an
        # expert's pairs are split evenly over its instances.  Real-time
        # planning on the exact loads is what `imbalance_after` reports.
        nc = np.asarray(wl.native_count); sc = np.asarray(wl.spare_count)
        slot_rank = np.repeat(np.arange(wl.num_ranks), nc + sc)
        p2l = plan.phy2log.cpu().numpy(); ld = load.cpu().numpy().astype(np.float64)
        stale = []
        for p in range(wl.layers, P):
            prev = p2l[p - wl.layers]
            used_slots = prev >= 0
            cnt = np.bincount(prev[used_slots], minlength=E)
            share = ld[p][prev[used_slots]] / cnt[prev[used_slots]]
            rank_load = np.bincount(slot_rank[used_slots], weights=share, minlength=wl.num_ranks)
            stale.append(rank_load.max() * wl.num_ranks / max(ld[p].sum(), 1.0))
        out["balance"]["previous_microbatch_placement_imbalance_mean"] = float(np.mean(stale))
        out["balance"]["previous_microbatch_placement_imbalance_max"] = float(np.max(stale))

    if args.cpu_budget > 0:
        ids_host = ids.cpu().numpy()
        cb, outs = cpu_baseline(ids_host, wl, args.cpu_budget)
        ok = True
        for p, (ld, pl, ph) in enumerate(outs):
            ok &= np.array_equal(load[p].cpu().numpy(), ld)
            ok &= np.array_equal(plan.phy2log[p].cpu().numpy(), pl.phy2log)
            ok &= np.array_equal(plan.phy_quota[p].cpu().numpy(), pl.phy_quota)
            ok &= np.array_equal(phys[p].cpu().numpy(), ph)
        out["cpu_baseline"] = cb
        out["parity_on_cpu_sample"] = bool(ok)
        # slot-count lower bound on the maximum rank load of the same layers
        # (no plan can beat it), as an imbalance, beside the planner's result
        from oracle.brute import slot_lower_bound
        lbs = []
        for p, (ld, _, _) in enumerate(outs):
            tot = int(ld.sum())
            if tot > 0:
                lam = slot_lower_bound(ld, wl.num_ranks, wl.num_spare)
                lbs.append((lam * wl.num_ranks / tot, float(imb_np[p, 1])))
        if lbs:
            lb = np.array(lbs)
            out["balance"]["lower_bound_layers"] = len(lbs)
            out["balance"]["imbalance_lower_bound_mean"] = float(lb[:, 0].mean())
            out["balance"]["imbalance_after_over_bound_max"] = float((lb[:, 1] / lb[:, 0]).max())
        cb["slot_fill"] = cpu_slot_fill(weights, plan.phy2log.cpu().numpy(), wl, min(args.cpu_budget, 5.0))
        cb["host_threads_available"] = os.cpu_count()
        cb["host_cpu"] = _cpu_model()
    else:
        out["cpu_baseline"] = None

    if args.workloads != "none":
        del ids, weights, slot, ws, phys, dpos, dsrc
        torch.cuda.empty_cache()
        names = [n for n in W.WORKLOAD_ORDER if n != wl.name] if args.workloads == "all" \
            else [n for n in args.workloads.split(",") if n]
        block = {wl.name: {
            "path_pairs_per_s": pairs_per_s, "path_ms": path_ms,
            "path_chunks": out["path_chunks"], "path_12B_frac": kern["path_frac"],
            "path_12B_frac_streaming_kernels": kern["path_stream_frac"],
            "hist_ms": ph_hist, "reroute_ms": ph_rr,
            "hist_rule_frac": kern["per_kernel"]["hist_rule_frac"],
            "reroute_rule_frac": kern["per_kernel"]["reroute_rule_frac"],
            "hist_moved_frac": kern["per_kernel"]["hist_moved_frac"],
            "reroute_moved_frac": kern["per_kernel"]["reroute_moved_frac"],
            "plan_us_per_layer_batched": ph_plan * 1e3 / P, "plan_us_single_layer": lat_plan,
            "dispatch_layout_ms": disp_ms,
            "dispatch_layout_12B_frac": next_rows["dispatch_layout_GBps"] / HBM_PEAK_GBPS,
            "fill_ms_per_layer": fill["ms"], "fill_frac": fill["frac"], "fill_moved_frac": fill["moved_frac"],
            "fill_layers": P, "filled_slots_mean": fill["filled"], "distinct_experts_mean": fill["distinct"],
            "imbalance_before_mean": out["balance"]["imbalance_before_mean"],
            "imbalance_after_mean": out["balance"]["imbalance_after_mean"],
            "imbalance_after_max": out["balance"]["imbalance_after_max"],
            "imbalance_lower_bound_mean": out["balance"].get("imbalance_lower_bound_mean"),
            "imbalance_after_over_bound_max": out["balance"].get("imbalance_after_over_bound_max"),
        }}
        for n in names:
            t0 = time.perf_counter()
            block[n] = workload_summary(n, dev, cpu_bound=args.cpu_budget > 0)
            print(f"[bench] workload {n}: {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
        out["workloads"] = block

    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
