"""Measure the cost model's constants on the GPU and write ``calib_gfx950.txt``.

    python -m reduce_scatter_amd.calibrate [--out PATH] [--quick]
    python -m reduce_scatter_amd.calibrate --schedules tree,dtree --ranks 32,72,128 --merge BASE [--out PATH]

The second form re-measures only the named schedules at the named rank counts
(after a change to the kernels that serve them) and keeps everything else from
the file BASE: the other schedules, and the named schedules' launch, step and
bandwidth constants and their other rank classes, so no rank class mixes
constants measured on two boxes; the new rank classes' latency terms and
corrections are fitted relative to BASE's constants.

The planner prices every legal schedule s of a call as

    t_s = launch_us[s] + step_us[s] * steps_s(n) + bytes_s / (bandwidth_s * corr_s[size bin])

("NCCL all-reduce" post, rakshithvasudev.github.io, section "How NCCL picks: a
cost model, not a threshold": latency plus bytes over bandwidth, argmin per
call, constants measured once; the tree's per-size correction table in the same
section is the model for ``corr``).  This script times every (collective,
schedule) over several rank counts and message sizes, fits launch_us, step_us
and bandwidth by least squares on relative error, then sets each size bin's
correction so the model matches the measured bandwidth-bound times.  Buffers
are torch device tensors (plumbing only); every timed call goes through the C
ABI, timed with HIP events on the launch stream.
"""
from __future__ import annotations

import argparse
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_OUT = os.path.join(HERE, "calib_gfx950.txt")
COLLS = ("allreduce", "reduce_scatter", "all_gather")
SCHEDS = ("ring", "tree", "fused", "split", "dtree")
SIZE_BINS = 48
HBM_BIN = 30                      # log2 of the footprint from which calls stream from HBM (1 GiB, 4x the MALL)


def _steps(coll, sched, n):
    if sched in ("fused", "split"):
        return 1
    if sched == "ring":
        return 2 * (n - 1) if coll == "allreduce" else n - 1
    depth = math.ceil(math.log2(n)) if n > 1 else 0              # depth of the bit-trick tree
    return 2 * depth


def rank_class(n):
    """The planner's rank class: ceil(log2 n), with 97-128 ranks a class (8) of
    their own apart from 65-96 (7)."""
    k = math.ceil(math.log2(n)) if n > 1 else 0
    return (8 if n > 96 else 7) if k >= 7 else k


def _bytes(coll, n, per_rank):
    """Algorithmic HBM bytes; per_rank = bytes of one rank's all-reduce buffer,
    reduce-scatter input or all-gather output."""
    return 2 * n * per_rank if coll == "allreduce" else (n + 1) * per_rank


def time_call(fn, iters, warmup=2):
    """Median GPU time (us) of one call, from an event pair around each call."""
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
    return float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))


def measure(ns, sizes, iters, rounds=3, dtype="f32", scheds=SCHEDS, colls=COLLS):
    """Time every (collective, schedule) at every rank count and per-rank byte
    size, for element type ``dtype`` (``f32`` or ``bf16``): median over
    ``rounds`` rounds of the per-call median of ``iters`` calls.  Only the
    schedules in ``scheds`` and the collectives in ``colls``."""
    import torch
    import reduce_scatter_amd as ar
    e = 4 if dtype == "f32" else 2
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    rows = []                                   # (coll, sched, n, per_rank_bytes, us)
    for n in ns:
        for size in sizes:
            # past 16 ranks, sizes of 3/4 of a power of two: buffers whose size and stride are powers of two put
            # the same offset of every rank on the same memory channels, which the split schedule (every rank at
            # one offset at a time) pays for and ranks do not in practice (gradient buckets have any size); at
            # 72 ranks on one box fused ran 2-4 % ahead of split at 2^22 elements per rank and 1-5 % behind at
            # the bucketed workload's sizes
            per_rank = size * 3 // 4 // 16 * 16 if n > 16 else size
            count = per_rank // e
            if count < n * (16 // e) or n * per_rank > (16 << 30):
                continue
            if n > 16:
                # many-rank all-reduces are gradient buckets: each rank's buffer a view into a larger flat gradient
                # buffer, reduced in place (see ar_out); on one box the all-reduce at 72 ranks ranked fused ahead
                # of split by 2 % with buffers of their own and split ahead by 4 % with views of a flat buffer
                flat_t = [torch.randn(2 * count + 1040, device="cuda").to(tdt) for _ in range(n)]
                xs_t = [f[count // 2 + 1040:count // 2 + 1040 + count] for f in flat_t]
            else:
                xs_t = [torch.randn(count, device="cuda").to(tdt) for _ in range(n)]
            ys_t = [torch.empty_like(x) for x in xs_t]
            R = count // n
            outs_t = [torch.empty(R, dtype=tdt, device="cuda") for _ in range(n)]
            # host pointer tables built once: the timings are the library's, not Python's marshalling
            xs, ys, outs = ar.pointers(xs_t), ar.pointers(ys_t), ar.pointers(outs_t)
            calls = {}
            # past 16 ranks the all-reduce is timed in place, on views of a flat gradient buffer (above)
            ar_out = xs if n > 16 else ys
            for sched in scheds:
                if "allreduce" in colls:
                    calls[("allreduce", sched)] = (
                        lambda s=sched: ar.ar_allreduce(xs, ar_out, count, dtype, "sum", n=n, sched=s))
                if sched in ("tree", "split", "dtree"):
                    continue
                if "reduce_scatter" in colls:
                    calls[("reduce_scatter", sched)] = (
                        lambda s=sched: ar.ar_reduce_scatter(xs, outs, R, dtype, "sum", n=n, sched=s))
                if "all_gather" in colls:
                    calls[("all_gather", sched)] = (lambda s=sched: ar.ar_all_gather(outs, ys, R, dtype, n=n, sched=s))
            # rounds that visit every call in turn, so no schedule always runs right after the same other one
            # (in the Infinity Cache regime the previous call's traffic decides what is cached)
            times = {k: [] for k in calls}
            for _ in range(rounds):
                for k, fn in calls.items():
                    times[k].append(time_call(fn, iters, warmup=1))
            for (coll, sched), v in times.items():
                rows.append((coll, sched, n, per_rank, float(np.median(v))))
            print("calibrate: %s n=%d %d bytes per rank done" % (dtype, n, per_rank), flush=True)
            del xs, ys, outs, xs_t, ys_t, outs_t
            flat_t = None
            torch.cuda.empty_cache()
    return rows


def fit(rows, latency=None, fixed=None):
    """Per (coll, sched): launch_us, step_us, bw_gbps, corr[SIZE_BINS].

    ``latency``: a fit of another element type whose launch, step and extra
    latency terms are kept (only the bandwidth terms are fitted here): the
    2-byte types share the 4-byte types' latency model.  ``fixed``:
    {(coll, sched): (launch_us, step_us, bw_gbps)} kept as given (launch and
    step ignored where ``latency`` has the entry); only the per-class terms
    are fitted, relative to them.

    Fitted by regime: launch and per-step costs from the calls that move at
    most 1 MB (pure latency: t = launch + step * steps), the sustained
    bandwidth from the calls that move at least 1 GB, then one correction per
    power-of-two footprint so the model meets the measured time wherever the
    bandwidth term is at least a quarter of it (footprints of 1 GB and more
    smoothed over neighbouring bins).  The footprint (total algorithmic bytes) is
    the size axis because it decides whether the data stays in the 256 MB
    Infinity Cache."""
    out = {}
    for coll in COLLS:
        for sched in SCHEDS:
            pts = [(n, pr, us, _bytes(coll, n, pr)) for c, s, n, pr, us in rows if c == coll and s == sched]
            if not pts:
                continue
            small_all = [(n, us) for n, pr, us, b in pts if b <= (1 << 20)]
            small = [(n, us) for n, us in small_all if n <= 16]    # the compile-time-n kernels
            keep = fixed.get((coll, sched)) if fixed else None
            if latency is not None and (coll, sched) in latency:
                launch, step, _, _, extra = latency[(coll, sched)]
            else:
                if keep is not None:
                    launch, step = keep[0], keep[1]
                elif sched in ("fused", "split") or len({n for n, _ in small}) < 2:
                    launch = float(np.median([us for _, us in small])) if small else 0.0
                    step = 0.0
                else:
                    A = np.array([[1.0, _steps(coll, sched, n)] for n, _ in small])
                    t = np.array([us for _, us in small])
                    (launch, step), *_ = np.linalg.lstsq(A, t, rcond=None)
                    launch, step = max(float(launch), 0.0), max(float(step), 0.0)
                extra = {}                                # rank class -> latency beyond launch + step * steps
                for rc in sorted({rank_class(n) for n, _ in small_all}):
                    res = [us - launch - step * _steps(coll, sched, n) for n, us in small_all
                           if rank_class(n) == rc]
                    if abs(float(np.median(res))) > 1.0:
                        extra[rc] = float(np.median(res))
            big = [(n, us, b) for n, pr, us, b in pts if b >= (1 << 30)]
            ref = big or [(n, us, b) for n, pr, us, b in pts]
            bws = [b / 1e3 / max(us - launch - step * _steps(coll, sched, n), 1e-3) for n, us, b in ref]
            bw = keep[2] if keep is not None else float(np.median(bws))
            corr = {}                                     # rank class -> [SIZE_BINS]
            per_bin = {}
            for n, pr, us, b in pts:
                term = us - launch - step * _steps(coll, sched, n) - extra.get(rank_class(n), 0.0)
                if term < 0.25 * us:                      # latency-bound: no bandwidth information
                    continue
                key = (rank_class(n), int(math.log2(b)))
                per_bin.setdefault(key, []).append(b / 1e3 / term / bw)
            for rc in sorted({k for k, _ in per_bin}):
                row = [1.0] * SIZE_BINS
                bins = {b: v for (k, b), v in per_bin.items() if k == rc}
                for b, v in bins.items():
                    row[b] = float(np.exp(np.mean(np.log(v))))
                top = max(bins)                           # beyond the largest measured footprint: keep its factor
                for b in range(top + 1, SIZE_BINS):
                    row[b] = row[top]
                # footprints of 1 GB and more stream from HBM: each keeps its own factor (the split kernel, for
                # one, slows at the largest footprints while the others do not), smoothed over its neighbouring
                # measured bins (median of three) so one noisy point does not flip a choice
                hb = sorted(b for b in bins if b >= HBM_BIN)
                sm = {}
                for i, b in enumerate(hb):
                    near = [row[x] for x in hb[max(0, i - 1):i + 2]]
                    sm[b] = float(np.median(near))
                for b, v in sm.items():
                    row[b] = v
                if hb:
                    for b in range(hb[-1] + 1, SIZE_BINS):
                        row[b] = sm[hb[-1]]
                corr[rc] = [min(4.0, max(0.05, c)) for c in row]
            out[(coll, sched)] = (launch, step, bw, corr, extra)
    return out


def entry_lines(model, model2=None):
    """The file's lines for each (collective, schedule) of ``model``."""
    out = {}
    for (coll, sched), (launch, step, bw, corr, extra) in sorted(model.items()):
        lines = ["%s %s %.3f %.4f %.1f" % (coll, sched, launch, step, bw)]
        for rc, row in sorted(corr.items()):
            lines.append("corr %s %s %d %s" % (coll, sched, rc, " ".join("%.3f" % c for c in row)))
        for rc, us in sorted(extra.items()):
            lines.append("lat %s %s %d %.3f" % (coll, sched, rc, us))
        if model2 and (coll, sched) in model2:
            _, _, bw2, corr2, _ = model2[(coll, sched)]
            lines.append("bw2 %s %s %.1f" % (coll, sched, bw2))
            for rc, row in sorted(corr2.items()):
                lines.append("corr2 %s %s %d %s" % (coll, sched, rc, " ".join("%.3f" % c for c in row)))
        out[(coll, sched)] = lines
    return out


def read_entries(path):
    """(header lines, {(collective, schedule): lines}) of a calibration file."""
    header, entries = [], {}
    for line in open(path):
        line = line.rstrip("\n")
        if not line.strip() or line.startswith("#"):
            header.append(line)
            continue
        tok = line.split()
        key = tuple(tok[1:3]) if tok[0] in ("corr", "lat", "bw2", "corr2") else tuple(tok[0:2])
        entries.setdefault(key, []).append(line)
    return header, entries


HEADER = ["# cost-model constants for libar (written by reduce_scatter_amd/calibrate.py)",
          None,
          "# <coll> <sched> <launch_us> <step_us> <bw_GBps>            (fitted on fp32: every 4-byte type)",
          "# corr <coll> <sched> <rank class: ceil(log2 n), 8 above 96> <bandwidth factor for log2(total algorithmic bytes) = 0..47>",
          "# lat <coll> <sched> <rank class> <latency beyond launch + step * steps, us>",
          "# bw2 / corr2: the same bandwidth terms fitted on bf16 (2-byte types; latency terms shared)"]


def base_constants(base):
    """{(coll, sched): (launch, step, bw)} and {(coll, sched): (launch, step,
    bw2)} of a calibration file as ``read_entries`` returns it."""
    four, two = {}, {}
    for key, lines in base[1].items():
        for line in lines:
            tok = line.split()
            if tok[0] == "bw2":
                two[key] = float(tok[3])
            elif tok[0] not in ("corr", "lat", "corr2"):
                four[key] = (float(tok[2]), float(tok[3]), float(tok[4]))
    return four, {k: (four[k][0], four[k][1], v) for k, v in two.items() if k in four}


def _row_class(line):
    """The rank class of a corr / corr2 / lat line, else None."""
    tok = line.split()
    return int(tok[3]) if tok[0] in ("corr", "lat", "corr2") else None


def write(path, model, gpu_name, model2=None, base=None, scheds=SCHEDS, classes=None, colls=COLLS):
    """The calibration file: ``model`` fitted on fp32 (every 4-byte type), and
    ``model2`` (bandwidth terms only) on bf16 for the 2-byte types.  With
    ``base`` (a calibration file as ``read_entries`` returns it), the entries
    of the schedules outside ``scheds`` are kept from it; with ``classes`` (rank
    classes ceil(log2 n)) as well, the named schedules keep BASE's lines too,
    except their latency and correction rows of those classes, which come from
    ``model`` (fitted relative to BASE's constants)."""
    entries = entry_lines(model, model2)
    header = [h if h is not None else "# device: %s" % gpu_name for h in HEADER]
    if base is not None:
        base_header, base_entries = base
        device = [h for h in base_header if h.startswith("# device:")]
        header[1] = device[0] if device else header[1]
        header += [h for h in base_header if h.startswith("# re-measured:")]
        where = "" if classes is None else " for rank classes %s" % ", ".join(str(c) for c in sorted(classes))
        what = ", ".join(scheds) if colls == COLLS else "%s %s" % ("/".join(colls), ", ".join(scheds))
        header.append("# re-measured: %s%s on %s" % (what, where, gpu_name))
        for key, lines in base_entries.items():
            if key[1] not in scheds or key not in entries:
                entries[key] = lines
            elif classes is not None:
                entries[key] = ([l for l in lines if _row_class(l) not in classes] +
                                [l for l in entries[key] if _row_class(l) in classes])
    with open(path, "w") as f:
        for h in header:
            f.write(h + "\n")
        for key in sorted(entries):
            for line in entries[key]:
                f.write(line + "\n")


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--out", default=DEFAULT_OUT)
    p.add_argument("--quick", action="store_true", help="fewer sizes and rank counts")
    p.add_argument("--schedules", default=",".join(SCHEDS), help="comma-separated schedules to measure")
    p.add_argument("--ranks", help="comma-separated rank counts to measure (default: all)")
    p.add_argument("--collectives", default=",".join(COLLS), help="comma-separated collectives to measure")
    p.add_argument("--merge", metavar="BASE", help="keep everything not re-measured from this file")
    a = p.parse_args(argv)
    scheds = tuple(x for x in a.schedules.split(",") if x)
    if not scheds or any(x not in SCHEDS for x in scheds):
        p.error("--schedules takes a comma-separated subset of %s" % ",".join(SCHEDS))
    colls = tuple(x for x in a.collectives.split(",") if x)
    if not colls or any(x not in COLLS for x in colls):
        p.error("--collectives takes a comma-separated subset of %s" % ",".join(COLLS))
    ranks = tuple(int(x) for x in a.ranks.split(",") if x) if a.ranks else None
    if ranks is not None and (not ranks or any(r < 2 or r > 128 for r in ranks)):
        p.error("--ranks takes rank counts from 2 to 128")
    if (scheds != SCHEDS or colls != COLLS or ranks is not None) and not a.merge:
        p.error("measuring a subset needs --merge BASE for the rest")
    import torch
    if not torch.cuda.is_available():
        print("calibrate: no GPU visible", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    ns = (2, 8) if a.quick else (2, 4, 8, 16, 32, 72, 128)
    sizes = [1 << k for k in ((12, 16, 20, 24, 28) if a.quick else (10, 12, 14, 16, 18, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30))]
    ns2 = (8,) if a.quick else (2, 4, 8, 16, 72)
    base = read_entries(a.merge) if a.merge else None   # read before --out may overwrite it
    fixed = fixed2 = classes = None
    if ranks is not None:
        ns, ns2 = ranks, tuple(r for r in ranks if r in ns2)
        classes = {rank_class(r) for r in ranks}
        fixed, fixed2 = base_constants(base)
    rows = measure(ns, sizes, iters=3 if a.quick else 5, scheds=scheds, colls=colls)
    model = fit(rows, fixed=fixed)
    rows2 = measure(ns2, sizes, iters=3 if a.quick else 5, dtype="bf16", scheds=scheds, colls=colls) if ns2 else []
    model2 = fit(rows2, latency=model, fixed=fixed2)
    gpu = torch.cuda.get_device_name(0) + " " + getattr(torch.cuda.get_device_properties(0), "gcnArchName", "")
    write(a.out, model, gpu, model2, base=base, scheds=scheds, classes=classes, colls=colls)
    for (coll, sched), (launch, step, bw, corr, extra) in sorted(model.items()):
        print("%-15s %-6s launch %7.2f us  step %6.3f us  bw %7.1f GB/s  extra %s" % (
            coll, sched, launch, step, bw, {k: round(v, 1) for k, v in extra.items()}))
    print("calibrate: wrote", a.out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
