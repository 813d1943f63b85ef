#!/usr/bin/env python3
"""Benchmark: all-reduce of n = 8 fp32 rank buffers of 256 MB each (64 Mi
elements per rank, N(0, 1e-3) synthetic gradients), all resident in one
MI355X's HBM.

One step = one ``ar_allreduce`` call through the C ABI with the schedule left
to the cost model (it plans, partitions, loads with the avg/sum pre-op, runs
the reduce-scatter hops, the postOp and the all-gather hops in one fused
pass).  The JSON line reports:

* ``value``: algbw = S / t_step (S = 256 MB per rank), GB/s (1e9 bytes/s);
* ``roofline``: the dominant kernel (the fused all-reduce) against HBM peak,
  ``achieved`` = 2*n*S algorithmic bytes / its average launch duration,
  timed with HIP events recorded on the launch stream around every launch;
  ``traffic`` = measured HBM bytes per launch from the committed counter
  summary when it was taken on the current kernel source, else null;
* ``cpu_baseline``: the CPU oracle on a bounded sample of the same workload;
* ``detail``: the other schedules and ops on the same buffers.

``--gpus N`` with N > 1 exits: the rank buffers live on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

N_RANKS = 8
COUNT = 64 << 20                      # fp32 elements per rank (256 MB)
PEAK_HBM_GBPS = 8000.0                # MI355X published HBM3E bandwidth
METRIC = "all-reduce algbw GB/s + % peak HBM BW (n=8, fp32, 256MB/rank)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_allreduce_n8_f32_256MB.traffic.json")
KERNEL_SRC = os.path.join(ROOT, "reduce_scatter_amd", "csrc", "fused.hip")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--op", default="sum", choices=["sum", "avg"])
    p.add_argument("--sched", default="auto", choices=["auto", "ring", "tree", "fused"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-detail", action="store_true")
    p.add_argument("--copy-probe", action="store_true",
                   help="time only a plain device copy of 2 GB (for HBM counter calibration) and exit")
    p.add_argument("--kernels", action="store_true",
                   help="instead of the JSON line, run each main kernel family 5 times at its workload's size and "
                        "print one JSON line per call (for kernel-trace and HBM-counter runs)")
    p.add_argument("--reshard", action="store_true",
                   help="instead of the JSON line, print the M-to-N reshard report (MoE layer, every route)")
    p.add_argument("--sweep", action="store_true",
                   help="instead of the JSON line, print a markdown report over every workload: the n=4 latency "
                        "case, the FSDP-shard reduce-scatter/all-gather, the n=16 int32 size sweep with the "
                        "planner's choice against the measured winner, and the 72-rank bucketed all-reduce")
    return p.parse_args()


# The kernel each schedule launches at this shape (n = 8, 16-byte aligned buffers).
KERNEL_OF = {"fused": "fused_allreduce_kernel", "ring": "ring_allreduce_fast", "tree": "tree_reg_kernel",
             "split": "split_allreduce_kernel", "dtree": "tree_reg_kernel"}


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, if it was
    taken on this exact kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def warm_up(fn, warmup, min_seconds=0.3):
    """At least ``warmup`` calls and at least ``min_seconds`` of them (wall
    clock, synchronised), so clocks and caches have settled whatever K/W are."""
    import torch
    t = time.perf_counter()
    calls = 0
    while calls < warmup or time.perf_counter() - t < min_seconds:
        fn()
        calls += 1
        if calls % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return calls


def time_region(fn, steps, stream):
    """``steps`` calls back to back between one pair of HIP events recorded on
    ``stream`` (the stream the kernels are launched on): the average time per
    call, with nothing recorded between the calls."""
    import torch
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def per_call_ms(fn, calls, stream):
    """One event pair around each call (diagnostics only: the events
    themselves add a few microseconds between calls)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def time_calls(fn, steps, warmup, stream):
    """Warm up, then the average time per call over ``steps`` calls (ms)."""
    warm_up(fn, warmup)
    return time_region(fn, steps, stream)


def copy_probe(args):
    import torch
    src = torch.empty(512 << 20, dtype=torch.float32, device="cuda")      # 2 GB
    dst = torch.empty_like(src)
    src.fill_(1.0)
    stream = torch.cuda.current_stream()
    launch_ms = time_calls(lambda: dst.copy_(src), args.steps, args.warmup, stream)
    print(json.dumps({"copy_probe_bytes_read": src.numel() * 4, "copy_probe_bytes_written": src.numel() * 4,
                      "launch_ms": round(launch_ms, 4),
                      "gbps": round(2 * src.numel() * 4 / (launch_ms * 1e-3) / 1e9, 1)}), flush=True)


def _interleaved_us(fns, rounds=3, iters=5):
    """Median GPU time (us) of each call in ``fns`` over ``rounds`` rounds that
    visit every call in turn (``iters`` timed calls each): no schedule is
    always the one that runs right after another's traffic or after the
    buffers were written."""
    import statistics
    times = {k: [] for k in fns}
    for _ in range(rounds):
        for k, fn in fns.items():
            times[k].append(_median_us(fn, iters=iters, warmup=1))
    return {k: statistics.median(v) for k, v in times.items()}


def kernel_calls(reps=5):
    """Each main kernel family at its workload's size, ``reps`` calls each,
    synchronised per call so a kernel trace or counter run sees whole,
    separate launches.  Prints the call, its kernel and its algorithmic
    bytes."""
    import torch
    import reduce_scatter_amd as ar
    import workloads as wl
    MB = 1 << 20

    def run(name, kernel, alg_bytes, fn):
        for _ in range(reps):
            fn()
            torch.cuda.synchronize()
        print(json.dumps({"call": name, "kernel": kernel, "algorithmic_bytes": alg_bytes, "calls": reps}), flush=True)

    n, C = N_RANKS, COUNT                                   # n = 8 fp32 all-reduce, 256 MB per rank
    xs_t = [wl.device_normal(1, 0, r, C, 1e-3, "f32") for r in range(n)]
    ys_t = [torch.empty(C, device="cuda") for _ in range(n)]
    xs, ys = ar.pointers(xs_t), ar.pointers(ys_t)
    for sched, kern in (("fused", "fused_allreduce_kernel"), ("ring", "ring_allreduce_fast"),
                        ("tree", "tree_reg_kernel"), ("dtree", "tree_reg_kernel"), ("split", "split_allreduce_kernel")):
        run("all-reduce n=8 f32 256MB/rank sum, %s" % sched, kern, 2 * n * C * 4,
            lambda: ar.ar_allreduce(xs, ys, C, "f32", "sum", sched=sched))
    del xs, ys, xs_t, ys_t
    R = 16 << 20                                            # FSDP shards: n = 8 bf16, 16 Mi elements per shard
    xs_t = [wl.device_normal(2, 0, r, n * R, 1e-2, "bf16") for r in range(n)]
    ys_t = [torch.empty(R, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    full_t = [torch.empty(n * R, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    xs, ys, full = ar.pointers(xs_t), ar.pointers(ys_t), ar.pointers(full_t)
    for r_, tag in ((R, ""), (R - 1, ", R-1 (phased)")):
        kern = "fused_reduce_scatter_kernel" if r_ == R else "fused_reduce_scatter_phased_kernel"
        run("reduce-scatter n=8 bf16 avg R=%d%s" % (r_, tag), kern, (n + 1) * n * r_ * 2,
            lambda: ar.ar_reduce_scatter(xs, ys, r_, "bf16", "avg", sched="fused"))
        kern = "fused_all_gather_kernel" if r_ == R else "fused_all_gather_phased_kernel"
        run("all-gather n=8 bf16 R=%d%s" % (r_, tag), kern, (n + 1) * n * r_ * 2,
            lambda: ar.ar_all_gather(ys, full, r_, "bf16", sched="fused"))
    del xs, ys, full, xs_t, ys_t, full_t
    n16, c16 = 16, 256 * MB // 4                            # the int32 sweep's ranks, 256 MB per rank
    xs_t = [torch.randint(-(1 << 20), 1 << 20, (c16,), dtype=torch.int32, device="cuda") for _ in range(n16)]
    ys_t = [torch.empty(c16, dtype=torch.int32, device="cuda") for _ in range(n16)]
    xs, ys = ar.pointers(xs_t), ar.pointers(ys_t)
    for sched, kern in (("fused", "fused_allreduce_kernel"), ("ring", "ring_allreduce_fast")):
        run("all-reduce n=16 i32 256MB/rank sum, %s" % sched, kern, 2 * n16 * c16 * 4,
            lambda: ar.ar_allreduce(xs, ys, c16, "i32", "sum", sched=sched))
    del xs, ys, xs_t, ys_t
    n72, c72 = 72, 25 * MB // 4                             # 72 ranks, one 25 MB fp32 bucket, in place
    bufs_t = [wl.device_normal(4, 1, r, c72, 1e-3, "f32") for r in range(n72)]
    bufs = ar.pointers(bufs_t)
    run("all-reduce n=72 f32 25MB/rank avg in place, split", "split_allreduce_kernel", 2 * n72 * c72 * 4,
        lambda: ar.ar_allreduce(bufs, bufs, c72, "f32", "avg", sched="split"))
    halves_rows(run, ar, bufs, 72, c72, "25MB")
    # the tree past 16 ranks: the streaming walk, then the LDS-staged kernels (each forced)
    run("all-reduce n=72 f32 25MB/rank avg in place, tree (streamed)", "tree_stream_kernel", 2 * n72 * c72 * 4,
        lambda: ar.ar_allreduce(bufs, bufs, c72, "f32", "avg", sched="tree"))
    os.environ["AR_TREE_STREAM"] = "0"
    for teams, kern in (("0", "tree_allreduce_kernel"), ("1", "tree_team_kernel")):
        os.environ["AR_TREE_TEAMS"] = teams
        run("all-reduce n=72 f32 25MB/rank avg in place, tree (staged, %s)" % ("teams" if teams == "1" else "level by level"),
            kern, 2 * n72 * c72 * 4, lambda: ar.ar_allreduce(bufs, bufs, c72, "f32", "avg", sched="tree"))
    os.environ.pop("AR_TREE_STREAM", None)
    del bufs, bufs_t
    n17, c17 = 17, 128 * MB // 4                            # 17 ranks, 128 MB per rank, in place
    bufs_t = [wl.device_normal(4, 1, r, c17, 1e-3, "f32") for r in range(n17)]
    bufs = ar.pointers(bufs_t)
    run("all-reduce n=17 f32 128MB/rank avg in place, tree (streamed)", "tree_stream_kernel", 2 * n17 * c17 * 4,
        lambda: ar.ar_allreduce(bufs, bufs, c17, "f32", "avg", sched="tree"))
    os.environ["AR_TREE_STREAM"] = "0"
    for teams, kern in (("0", "tree_allreduce_kernel"), ("1", "tree_team_kernel")):
        os.environ["AR_TREE_TEAMS"] = teams
        run("all-reduce n=17 f32 128MB/rank avg in place, tree (staged, %s)" % ("teams" if teams == "1" else "level by level"),
            kern, 2 * n17 * c17 * 4, lambda: ar.ar_allreduce(bufs, bufs, c17, "f32", "avg", sched="tree"))
    os.environ.pop("AR_TREE_TEAMS", None)
    os.environ.pop("AR_TREE_STREAM", None)
    del bufs, bufs_t
    n128, c128 = 128, 8 * MB // 4                           # 128 ranks, 8 MB per rank, in place
    bufs_t = [wl.device_normal(4, 2, r, c128, 1e-3, "f32") for r in range(n128)]
    bufs = ar.pointers(bufs_t)
    for sched, kern in (("tree", "tree_stream_kernel"), ("split", "split_allreduce_kernel")):
        run("all-reduce n=128 f32 8MB/rank avg in place, %s" % sched, kern, 2 * n128 * c128 * 4,
            lambda: ar.ar_allreduce(bufs, bufs, c128, "f32", "avg", sched=sched))
    halves_rows(run, ar, bufs, 128, c128, "8MB")
    del bufs, bufs_t
    torch.cuda.empty_cache()


def halves_rows(run, ar, bufs, n, count, size):
    """The fused schedule past 16 ranks: its reduce-scatter and all-gather halves (one call launches both; each
    kernel's row carries its own algorithmic bytes: (n+1)*S, then S read and (n-1)*S written), then the wide
    one-pass kernel (AR_AR_HALVES=0, 2*n*S)."""
    S = count * 4
    run("all-reduce n=%d f32 %s/rank avg in place, fused (reduce-scatter half, all-gather half)" % (n, size),
        ["fused_reduce_scatter_phased_kernel", "allreduce_chunk_gather_kernel"], [(n + 1) * S, n * S],
        lambda: ar.ar_allreduce(bufs, bufs, count, "f32", "avg", sched="fused"))
    os.environ["AR_AR_HALVES"] = "0"
    run("all-reduce n=%d f32 %s/rank avg in place, fused (one pass)" % (n, size), "fused_allreduce_wide_kernel",
        2 * n * S, lambda: ar.ar_allreduce(bufs, bufs, count, "f32", "avg", sched="fused"))
    os.environ.pop("AR_AR_HALVES", None)


def _median_us(fn, iters=10, warmup=2):
    import statistics
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) * 1e3 for a, b in ev)


def sweep():
    """Markdown report over every workload (GPU times: median of per-call HIP event pairs)."""
    import torch
    import reduce_scatter_amd as ar
    import workloads as wl
    out = ["# Workload sweep (MI355X)", "", "Command: `python bench.py --sweep` (from the repository root).", "",
           "GPU time per call = median over 10 calls of an event pair around each call; "
           "HBM GB/s = algorithmic bytes / time; % of the 8 TB/s peak.", ""]

    # n = 4, fp32, 1024 elements: the latency regime
    xs = [torch.from_numpy(x).cuda() for x in wl.c1_inputs()]
    ys = [torch.empty_like(x) for x in xs]
    xs, ys = ar.pointers(xs), ar.pointers(ys)          # host pointer tables built once, outside the timing
    out += ["## n = 4, fp32, 1024 elements per rank (latency regime)", "", "| call (all-reduce unless named) | us |",
            "|---|---|"]
    for sched in ("fused", "ring", "tree", "split", "dtree", "auto"):
        out.append("| %s | %.2f |" % (sched, _median_us(lambda: ar.ar_allreduce(xs, ys, 1024, "f32", "sum", sched=sched))))
    # the same call captured 100 times into one HIP graph (torch's graph API): GPU time per call without the
    # host's per-call cost
    reps = 100
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ar.ar_allreduce(xs, ys, 1024, "f32", "sum", sched="fused")
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            ar.ar_allreduce(xs, ys, 1024, "f32", "sum", sched="fused")
    out.append("| fused, %d calls replayed from one HIP graph (per call) | %.2f |" % (
        reps, _median_us(graph.replay, iters=5) / reps))
    del graph
    # the c1 reduce-scatter of the same inputs (256 elements out per rank) and the all-gather of its outputs
    outs_t = [torch.empty(256, device="cuda") for _ in range(4)]
    outs = ar.pointers(outs_t)
    for sched in ("fused", "ring"):
        out.append("| reduce-scatter (%s), 256 elements out per rank | %.2f |" % (
            sched, _median_us(lambda: ar.ar_reduce_scatter(xs, outs, 256, "f32", "sum", sched=sched))))
        out.append("| all-gather (%s), 256 elements in per rank | %.2f |" % (
            sched, _median_us(lambda: ar.ar_all_gather(outs, ys, 256, "f32", sched=sched))))
    out.append("")

    # FSDP shards: reduce-scatter (avg) of 8 x 128 Mi bf16, all-gather of 8 x 16 Mi bf16
    n, R = 8, 16 << 20
    xs_t = [wl.device_normal(2, 0, r, n * R, 1e-2, "bf16") for r in range(n)]
    ys_t = [torch.empty(R, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    xs, ys = ar.pointers(xs_t), ar.pointers(ys_t)
    out += ["## FSDP shards, n = 8, bf16: reduce-scatter (avg) 256 MB in per rank; all-gather 32 MB in per rank", "",
            "| call | schedule | us | HBM GB/s | % peak |", "|---|---|---|---|---|"]
    alg = (n + 1) * n * R * 2
    for sched in ("fused", "ring"):
        us = _median_us(lambda: ar.ar_reduce_scatter(xs, ys, R, "bf16", "avg", sched=sched))
        out.append("| reduce-scatter | %s | %.1f | %.0f | %.1f |" % (sched, us, alg / us / 1e3, alg / us / 1e3 / PEAK_HBM_GBPS * 100))
    # reducing in fp32: fp32 partials over the bf16 buffers, against a reduce-scatter of fp32 copies
    us = _median_us(lambda: ar.ar_reduce_scatter_ex(xs, ys, R, "bf16", "avg", sched="fused", acc="fp32"))
    out.append("| reduce-scatter, fp32 partials (bf16 in and out) | fused | %.1f | %.0f | %.1f |" % (
        us, alg / us / 1e3, alg / us / 1e3 / PEAK_HBM_GBPS * 100))
    # an odd shard length: slices of R - 1 elements (not whole 16-byte vectors: the phased pass)
    R1, alg1 = R - 1, (n + 1) * n * (R - 1) * 2
    us = _median_us(lambda: ar.ar_reduce_scatter(xs, ys, R1, "bf16", "avg", sched="fused"))
    out.append("| reduce-scatter, R - 1 elements per slice (phased) | fused | %.1f | %.0f | %.1f |" % (
        us, alg1 / us / 1e3, alg1 / us / 1e3 / PEAK_HBM_GBPS * 100))
    x32_t = [x.float() for x in xs_t]
    y32_t = [torch.empty(R, device="cuda") for _ in range(n)]
    x32, y32 = ar.pointers(x32_t), ar.pointers(y32_t)
    us32 = _median_us(lambda: ar.ar_reduce_scatter(x32, y32, R, "f32", "avg", sched="fused"))
    out.append("| reduce-scatter of fp32 copies (twice the bytes; the cast not timed) | fused | %.1f | %.0f | %.1f |" % (
        us32, 2 * alg / us32 / 1e3, 2 * alg / us32 / 1e3 / PEAK_HBM_GBPS * 100))
    del x32, y32, x32_t, y32_t
    del xs, xs_t
    pieces_t = [wl.device_uniform(2, 1, r, R, -1.0, 1.0, "bf16") for r in range(n)]
    full_t = [torch.empty(n * R, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    pieces, full = ar.pointers(pieces_t), ar.pointers(full_t)
    for sched in ("fused", "ring"):
        us = _median_us(lambda: ar.ar_all_gather(pieces, full, R, "bf16", sched=sched))
        out.append("| all-gather | %s | %.1f | %.0f | %.1f |" % (sched, us, alg / us / 1e3, alg / us / 1e3 / PEAK_HBM_GBPS * 100))
    us = _median_us(lambda: ar.ar_all_gather(pieces, full, R1, "bf16", sched="fused"))
    out.append("| all-gather, R - 1 elements per piece (phased) | fused | %.1f | %.0f | %.1f |" % (
        us, alg1 / us / 1e3, alg1 / us / 1e3 / PEAK_HBM_GBPS * 100))
    del pieces, full, ys, pieces_t, full_t, ys_t
    torch.cuda.empty_cache()
    out.append("")

    # n = 16 int32 size sweep: every schedule, the planner's choice and the measured winner
    n = wl.C4_N
    out += ["## n = 16, int32, 1 KB .. 1 GB per rank: schedules, planner choice, measured winner", "",
            "Regime: n*S <= 256 MB fits the MI355X's 256 MB Infinity Cache (latency/cache regime); larger is HBM.", "",
            "| bytes/rank | op | ring us | tree us | dtree us | fused us | split us | planner | winner | toll % | best HBM GB/s "
            "| regime |", "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    agree = cells = near = 0
    for size in wl.C4_SIZES:
        count = size // 4
        xs_t = [wl.device_ints(3, int(np.log2(size)), r, count, -(1 << 20), 1 << 20, "i32") for r in range(n)]
        ys_t = [torch.empty_like(x) for x in xs_t]
        xs, ys = ar.pointers(xs_t), ar.pointers(ys_t)
        for op in ("sum", "min", "max", "avg"):
            t = _interleaved_us({s: (lambda s=s: ar.ar_allreduce(xs, ys, count, "i32", op, n=n, sched=s))
                                 for s in ("ring", "tree", "dtree", "fused", "split")}, rounds=5, iters=8)
            plan = ar.ar_plan("allreduce", count, "i32", op, n).chosen
            win = min(t, key=t.get)
            toll = 100.0 * (t[plan] / t[win] - 1.0)
            cells += 1
            agree += plan == win
            near += toll <= 5.0
            out.append("| %d | %s | %.1f | %.1f | %.1f | %.1f | %.1f | %s | %s | %.1f | %.0f | %s |" % (
                size, op, t["ring"], t["tree"], t["dtree"], t["fused"], t["split"], plan, win, toll,
                2 * n * size / t[win] / 1e3,
                "cache" if n * size <= (256 << 20) else "HBM"))
        del xs, ys, xs_t, ys_t
        torch.cuda.empty_cache()
    out += ["", "Planner agreed with the measured winner in %d of %d cells; its choice was within 5 %% of the "
            "winner's time in %d of %d (below 1 MB per rank the schedules differ by less than the run-to-run "
            "noise of about 1 us)." % (agree, cells, near, cells), ""]

    # 72 ranks, gradient buckets, avg, in place, back to back on one stream
    n = wl.C5_N
    buckets, total = wl.c5_buckets()
    grads = [wl.device_spiky_normal(4, r, total // 4, 1e-3, 0.01, 100.0) for r in range(n)]
    views = [(ar.pointers([g[off // 4:(off + nb) // 4] for g in grads]), nb // 4) for off, nb in buckets]

    def all_buckets(sched):
        for v, c in views:
            ar.ar_allreduce(v, v, c, "f32", "avg", n=n, sched=sched)
    alg = 2 * n * total
    out += ["## 72 ranks, fp32 avg, %d gradient buckets (%.1f MB per rank), in place, back to back" % (len(buckets), total / 2**20), "",
            "| schedule | total per sweep (us) | effective HBM GB/s (2*72*bytes / t) | % of peak | per bucket us: min / median / max |",
            "|---|---|---|---|---|"]
    for sched in ("auto", "split", "fused"):
        us = _median_us(lambda: all_buckets(sched), iters=5, warmup=1)
        per = sorted(_median_us(lambda v=v, c=c: ar.ar_allreduce(v, v, c, "f32", "avg", n=n, sched=sched), iters=5, warmup=1)
                     for v, c in views)
        out.append("| %s | %.1f | %.0f | %.1f | %.1f / %.1f / %.1f |" % (
            sched, us, alg / us / 1e3, alg / us / 1e3 / PEAK_HBM_GBPS * 100, per[0], per[len(per) // 2], per[-1]))
    out += ["", "Planner choice for a 25 MB bucket: %s." % ar.ar_plan("allreduce", (25 << 20) // 4, "f32", "avg", n).chosen, ""]
    del grads, views
    torch.cuda.empty_cache()
    out += reshard_report()
    out += cpu_report()
    print("\n".join(out), flush=True)


def reshard_report():
    """The M-to-N reshard of the NCCL M2N paper's single-layer microbenchmark
    on one GPU: a [256, 2048, 7168] bf16 tensor (7168 MB) from 16 EP shards
    (Shard(0)) to TP8 x DP r_d (Shard(1), r_d replicas), every route.  HBM
    GB/s = the route's own bytes / time; "vs fused bound" = (1 + r_d) * B /
    time, B the unique payload (each source byte read once, each destination
    byte written once)."""
    import torch
    import reduce_scatter_amd as ar
    S = (256, 2048, 7168)
    src = ar.Layout(S, (1, 16), (ar.REPLICATE, 0), 0)
    src_t = [torch.empty(ar.local_shape(src, s), dtype=torch.bfloat16, device="cuda").uniform_(-1, 1)
             for s in range(16)]
    out = ["## M-to-N reshard, [256, 2048, 7168] bf16 (7168 MB), 16 EP shards -> TP8 x DP r_d, one GPU", "",
           "| r_d | route | ms | route bytes (GB) | HBM GB/s | % peak | vs fused bound GB/s | planner |",
           "|---|---|---|---|---|---|---|---|"]
    for rd in (2, 4, 8):
        dst = ar.Layout(S, (rd, 8), (ar.REPLICATE, 1), 16)
        dst_t = [torch.empty(ar.local_shape(dst, t), dtype=torch.bfloat16, device="cuda") for t in range(8 * rd)]
        sp, dp = ar.pointers(src_t), ar.pointers(dst_t)
        plan = ar.ar_reshard_plan(src, dst, 2)
        bound = (1 + rd) * plan.unique_bytes
        for route in ("flat", "hier", "fused"):
            us = _median_us(lambda: ar.ar_reshard(sp, dp, src, dst, 2, route=route), iters=5, warmup=1)
            b = plan.bytes[route]
            out.append("| %d | %s | %.3f | %.1f | %.0f | %.1f | %.0f | %s |" % (
                rd, route, us / 1e3, b / 1e9, b / us / 1e3, b / us / 1e3 / PEAK_HBM_GBPS * 100, bound / us / 1e3,
                "chosen" if plan.chosen == route else ""))
        del dst_t, dp
        torch.cuda.empty_cache()
    out.append("")
    return out


def cpu_baseline(min_seconds=10.0):
    """The oracle, as it stands, on the benchmark's own workload: the ring
    all-reduce (sum) of n = 8 ranks of 64 Mi fp32 elements (256 MB each),
    N(0, 1e-3) host data (torch's CPU generator with the device buffers'
    seeds).  One call warms the host allocator; then calls are timed until at
    least ``min_seconds`` of CPU work have run.  ``value`` is algbw (256 MB
    per rank / mean time per call), the metric's own unit; ``hbm_equiv_GBps``
    is the algorithmic bytes 2*n*S / time, the figure the GPU's roofline uses."""
    import oracle
    import workloads
    count = COUNT
    xs = [workloads.device_normal(1, 0, r, count, 1e-3, "f32", device="cpu").numpy() for r in range(N_RANKS)]
    out = [np.empty_like(x) for x in xs]
    oracle.ring_allreduce(xs, "f32", "sum", out=out)
    calls = 0
    t = time.perf_counter()
    while True:
        oracle.ring_allreduce(xs, "f32", "sum", out=out)
        calls += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds:
            break
    per = dt / calls
    return {"value": round(count * 4 / per / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "hbm_equiv_GBps": round(2 * N_RANKS * count * 4 / per / 1e9, 3),
            "sample": "the whole workload: ring all-reduce (sum), n=8, fp32, 64 Mi elements (256 MB) per rank, "
                      "%d calls in %.1f s (%.2f s per call)" % (calls, dt, per)}


def cpu_baseline_one_core(min_seconds=4.0):
    """The same oracle call at one thread on a bounded sample (the first
    1/16 of every rank buffer), timed until ``min_seconds`` have run."""
    import oracle
    import workloads
    count = COUNT // 16
    xs = [workloads.device_normal(1, 0, r, COUNT, 1e-3, "f32", device="cpu").numpy()[:count].copy()
          for r in range(N_RANKS)]
    out = [np.empty_like(x) for x in xs]
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        oracle.ring_allreduce(xs, "f32", "sum", out=out)
        calls, t = 0, time.perf_counter()
        while True:
            oracle.ring_allreduce(xs, "f32", "sum", out=out)
            calls += 1
            dt = time.perf_counter() - t
            if dt >= min_seconds:
                break
    finally:
        oracle.set_num_threads(threads)
    per = dt / calls
    return {"value": round(count * 4 / per / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "cpu_model": cpu_model(), "hbm_equiv_GBps": round(2 * N_RANKS * count * 4 / per / 1e9, 3),
            "sample": "ring all-reduce (sum), n=8, fp32, the first 4 Mi elements (16 MB) of every rank, "
                      "%d calls in %.1f s" % (calls, dt)}


def _cpu_time(fn, min_seconds):
    """Mean wall time per call (s) of ``fn`` after one warm-up call, over at
    least ``min_seconds``."""
    fn()
    calls, t = 0, time.perf_counter()
    while True:
        fn()
        calls += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds:
            return dt / calls, calls


def cpu_report(min_seconds=2.0):
    """The oracle, as it stands, on every workload (bounded samples of the
    large ones), at all host threads and at one: time per call and GB/s of
    algorithmic bytes (all-reduce 2*n*S, reduce-scatter and all-gather
    (n+1)*n*R*e).  A baseline beside the GPU numbers, not a target."""
    import oracle
    import workloads as wl
    MB = 1 << 20
    threads = oracle.num_threads()
    rows = []

    def c1():
        xs = wl.c1_inputs()
        return (lambda: oracle.ring_allreduce(xs, "f32", "sum")), 2 * 4 * 1024 * 4, \
            "all-reduce sum, n=4, fp32, 1024 elements per rank (the whole workload)"

    def c2():
        c = 8 * MB
        xs = [wl.normal(1, 0, r, c, 1e-3, "f32") for r in range(8)]
        return (lambda: oracle.ring_allreduce(xs, "f32", "sum")), 2 * 8 * c * 4, \
            "all-reduce sum, n=8, fp32, 8 Mi elements (32 MB) per rank: 1/8 of the 256 MB per rank workload"

    def c3_rs():
        R = 2 * MB
        xs = [wl.normal(2, 0, r, 8 * R, 1e-2, "bf16") for r in range(8)]
        return (lambda: oracle.ring_reduce_scatter(xs, "bf16", "avg")), 9 * 8 * R * 2, \
            "reduce-scatter avg, n=8, bf16, 2 Mi elements out per rank (16 Mi in): 1/8 of the FSDP shard"

    def c3_ag():
        R = 2 * MB
        xs = [wl.uniform(2, 1, r, R, -1.0, 1.0, "bf16") for r in range(8)]
        return (lambda: oracle.ring_all_gather(xs, "bf16")), 9 * 8 * R * 2, \
            "all-gather, n=8, bf16, 2 Mi elements in per rank: 1/8 of the FSDP shard"

    def c4():
        c = 4 * MB
        xs = [wl.ints(3, 30, r, c, -(1 << 20), 1 << 20, "i32") for r in range(16)]
        return (lambda: oracle.ring_allreduce(xs, "i32", "sum")), 2 * 16 * c * 4, \
            "all-reduce sum, n=16, int32, 4 Mi elements (16 MB) per rank: 1/64 of the 1 GB per rank cell"

    def c5():
        buckets, _ = wl.c5_buckets()
        c = buckets[0][1] // 4 // 4
        xs = [wl.normal(4, 1, r, c, 1e-3, "f32") for r in range(72)]
        return (lambda: oracle.pairwise_reduce(xs, "f32", "avg")), 2 * 72 * c * 4, \
            "all-reduce avg, n=72, fp32, the pairwise order the planner picks, %d elements per rank: a quarter " \
            "of the first 25 MB bucket" % c

    for name, make in (("c1", c1), ("c2", c2), ("c3 reduce-scatter", c3_rs), ("c3 all-gather", c3_ag), ("c4", c4),
                       ("c5", c5)):
        fn, alg, sample = make()
        per_all, calls_all = _cpu_time(fn, min_seconds)
        oracle.set_num_threads(1)
        try:
            per_one, calls_one = _cpu_time(fn, min_seconds)
        finally:
            oracle.set_num_threads(threads)
        rows.append((name, sample, per_all, alg / per_all / 1e9, per_one, alg / per_one / 1e9))
        del fn
    out = ["## CPU oracle on every workload (a baseline, not the target)", "",
           "Host: %s, %d threads (OpenMP over the elements of each message; results identical at any thread "
           "count). Time per call after one warm-up call, at least %.0f s of calls per cell; GB/s = algorithmic "
           "bytes (all-reduce 2*n*S; reduce-scatter / all-gather (n+1)*n*R*e) / time." % (cpu_model(), threads,
                                                                                         min_seconds), "",
           "| workload | sample | ms per call, %d threads | GB/s | ms per call, 1 thread | GB/s |" % threads,
           "|---|---|---|---|---|---|"]
    for name, sample, pa, ga, po, go in rows:
        out.append("| %s | %s | %.3f | %.3f | %.3f | %.3f |" % (name, sample, pa * 1e3, ga, po * 1e3, go))
    out.append("")
    return out


def copy_ceiling(stream, alg_bytes):
    """A plain device copy moving the same bytes as one all-reduce (half read,
    half written): the library's all-gather over one rank, one 16-byte load
    and one store per lane (the runtime's own device-to-device copy runs at
    about 4.6-4.8 TB/s on MI355X, well below it) -- the practical ceiling of
    the read/write mix."""
    import torch
    import reduce_scatter_amd as ar
    src = torch.empty(alg_bytes // 8, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    S, D = ar.pointers([src]), ar.pointers([dst])
    ms = time_calls(lambda: ar.ar_all_gather(S, D, src.numel(), "f32", n=1, sched="fused", stream=stream), 10, 2, stream)
    del src, dst
    return {"bytes": alg_bytes, "ms": round(ms, 4), "GBps": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
            "frac": round(alg_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}


def cpu_model() -> str:
    """The host CPU's model name (as lscpu reports it, read from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this workload keeps all %d logical ranks in ONE GPU's HBM; "
              "runs on more than one GPU are not part of it (got --gpus %d)" % (N_RANKS, args.gpus),
              file=sys.stderr)
        return 2
    if args.steps < 1:
        print("--steps must be >= 1", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args)
        return 0
    if args.kernels:
        kernel_calls()
        return 0
    if args.sweep:
        sweep()
        return 0
    if args.reshard:
        print("\n".join(reshard_report()), flush=True)
        return 0

    import reduce_scatter_amd as ar
    import workloads

    stream = torch.cuda.current_stream()
    xs_t = [workloads.device_normal(1, 0, r, COUNT, 1e-3, "f32") for r in range(N_RANKS)]
    ys_t = [torch.empty_like(x) for x in xs_t]
    xs, ys = ar.pointers(xs_t), ar.pointers(ys_t)       # the rank pointer tables, built once
    torch.cuda.synchronize()
    S = COUNT * 4
    alg_bytes = 2 * N_RANKS * S

    def step():
        ar.ar_allreduce(xs, ys, COUNT, "f32", args.op, sched=args.sched, stream=stream)

    plan = ar.ar_plan("allreduce", COUNT, "f32", args.op, N_RANKS)
    chosen = plan.chosen if args.sched == "auto" else args.sched
    warm_calls = warm_up(step, args.warmup)
    # The timed region: K steps back to back between one event pair on the launch stream.  Each step is one
    # launch of the schedule's kernel, so the average launch duration over the region is the time per step,
    # and ``value``, the roofline and the % of peak all use this one denominator.
    step_ms = time_region(step, args.steps, stream)
    algbw = S / (step_ms * 1e-3) / 1e9
    achieved = alg_bytes / (step_ms * 1e-3) / 1e9
    # Diagnostics after the timed region: one event pair around each of K more calls.
    per = per_call_ms(step, args.steps, stream)
    per_sorted = sorted(per)

    detail = {}
    if not args.no_detail:
        for sched in ("fused", "ring", "tree", "split", "dtree"):
            for op in ("sum", "avg"):
                lms = time_calls(
                    lambda: ar.ar_allreduce(xs, ys, COUNT, "f32", op, sched=sched, stream=stream), 10, 2, stream)
                detail["%s_%s" % (sched, op)] = {"ms": round(lms, 4),
                                                 "algbw_GBps": round(S / (lms * 1e-3) / 1e9, 1),
                                                 "hbm_GBps": round(alg_bytes / (lms * 1e-3) / 1e9, 1)}
        detail["planner"] = {"chosen": plan.chosen, "predicted_us": {k: round(v, 1) for k, v in
                                                                    plan.predicted_us.items()}}
        cc = copy_ceiling(stream, alg_bytes)
        cc["fused_over_copy"] = round(cc["ms"] / step_ms, 4) if chosen == "fused" else None
        detail["copy_ceiling"] = cc

    out = {
        "metric": METRIC,
        "value": round(algbw, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "all-reduce, n=8 logical ranks on one GPU, fp32, 64Mi elements (256 MB) per rank, "
                               "N(0,1e-3), op=%s, schedule=%s (%s), out of place" % (args.op, args.sched, chosen),
                   "n_ranks": N_RANKS, "count_per_rank": COUNT, "bytes_per_rank": S, "op": args.op,
                   "schedule": chosen},
        "hbm_GBps": round(achieved, 1),
        "pct_peak_hbm": round(100.0 * achieved / PEAK_HBM_GBPS, 2),
        "busbw_GBps": round(algbw * 2 * (N_RANKS - 1) / N_RANKS, 2),
        "roofline": {"bound": "hbm", "kernel": "%s<f32,%s>" % (KERNEL_OF[chosen], args.op),
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic() if chosen == "fused" else None,
                     "algorithmic_bytes_per_launch": alg_bytes, "avg_launch_ms": round(step_ms, 4),
                     "avg_launch_ms_from": "the timed region: %d launches back to back between one event pair on "
                                           "the launch stream" % args.steps,
                     "per_call_events_ms": {"calls": len(per), "median": round(per_sorted[len(per) // 2], 4),
                                            "min": round(per_sorted[0], 4), "first": round(per[0], 4),
                                            "last": round(per[-1], 4)},
                     "warmup_calls": warm_calls},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(),
        "detail": detail,
    }
    if not args.no_cpu_baseline and not args.no_detail:
        detail["cpu_baseline_one_core"] = cpu_baseline_one_core()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
