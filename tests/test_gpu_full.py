"""Parity at the benchmark workloads' full sizes, in the launch configuration
``bench.py`` times (default schedule choice and residency caps).

* 8 ranks x 256 MB fp32 (sum, avg; fused, ring, tree; in and out of place):
  every output element against the ring / tree oracle.
* FSDP-style shards: reduce-scatter (avg) of 8 x 128 Mi bf16 and all-gather
  of 8 x 16 Mi bf16: every element against the oracle.
* n = 16 int32 sweep, 1 KB .. 1 GB per rank: every op and schedule, every
  element of every rank against the oracle (int32 sums wrap exactly, so the
  plain element-wise definition is exact; computed in streamed slices).
* 72 ranks, 29 gradient buckets of up to 25 MB packed from 256 tensors, avg,
  in place, back to back: every bucket of every rank checked (ranks agree on
  the device, rank 0 against the oracle of the planner's choice); the split
  schedule on one 25 MB bucket against the pairwise oracle.
* The split schedule at the 8 x 256 MB shape against the pairwise oracle.
* Past every 32-bit byte offset: n = 2 fp32 all-reduce of 4.3 GB per rank
  (every schedule), reduce-scatter and all-gather of 4.3 GB slices: every
  element checked on the device (n = 2 is one IEEE operation per element),
  sampled windows against the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from devutil import assert_bits_equal, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
ar = pytest.importorskip("reduce_scatter_amd")

MB = 1 << 20


def _same_on_all_ranks(ys):
    """Every rank holds the identical result (compared bit for bit on the device)."""
    for y in ys[1:]:
        assert torch.equal(y.view(torch.uint8), ys[0].view(torch.uint8)), "ranks disagree"


@pytest.fixture(scope="module")
def c2_inputs():
    n, count = 8, 64 * MB
    xs = [workloads.device_normal(1, 0, r, count, 1e-3, "f32") for r in range(n)]
    host = [to_host(x, "f32") for x in xs]
    yield xs, host
    del xs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("op", ["sum", "avg"])
def test_c2_fused_and_ring_full_size(c2_inputs, op):
    xs, host = c2_inputs
    count = xs[0].numel()
    print("c2 oracle", op, flush=True)
    want = oracle.ring_allreduce(host, "f32", op)[0]
    assert ar.ar_plan("allreduce", count, "f32", op, 8).chosen in ("fused", "ring")    # ring hop order
    for sched in ("auto", "fused", "ring"):
        print("c2", op, sched, flush=True)
        ys = [torch.empty_like(x) for x in xs]
        ar.ar_allreduce(xs, ys, count, "f32", op, sched=sched)
        torch.cuda.synchronize()
        _same_on_all_ranks(ys)
        assert_bits_equal(to_host(ys[0], "f32"), want, "c2 %s %s" % (op, sched))
        del ys


def test_c2_split_full_size(c2_inputs):
    xs, host = c2_inputs
    count = xs[0].numel()
    print("c2 split oracle", flush=True)
    want = oracle.pairwise_reduce(host, "f32", "sum")
    ys = [torch.empty_like(x) for x in xs]
    ar.ar_allreduce(xs, ys, count, "f32", "sum", sched="split")
    torch.cuda.synchronize()
    _same_on_all_ranks(ys)
    got = to_host(ys[0], "f32")
    assert_bits_equal(got, want, "c2 split")
    ring = oracle.ring_allreduce(host, "f32", "sum")[0]
    assert np.max(np.abs(got.astype(np.float64) - ring)) <= 1e-6 * np.max(np.abs(ring))


def test_c2_tree_and_in_place_full_size(c2_inputs):
    xs, host = c2_inputs
    count = xs[0].numel()
    print("c2 tree oracle", flush=True)
    want_tree = oracle.tree_allreduce(host, "f32", "sum")[0]
    ys = [torch.empty_like(x) for x in xs]
    ar.ar_allreduce(xs, ys, count, "f32", "sum", sched="tree")
    torch.cuda.synchronize()
    _same_on_all_ranks(ys)
    got = to_host(ys[0], "f32")
    assert_bits_equal(got, want_tree, "c2 tree")
    print("c2 dtree oracle", flush=True)
    want_dtree = oracle.dtree_allreduce(host, "f32", "sum")[0]
    ar.ar_allreduce(xs, ys, count, "f32", "sum", sched="dtree")
    torch.cuda.synchronize()
    _same_on_all_ranks(ys)
    assert_bits_equal(to_host(ys[0], "f32"), want_dtree, "c2 dtree")
    ring = oracle.ring_allreduce(host, "f32", "sum")[0]
    # the tree's order differs from the ring's: normwise 1e-6
    assert np.max(np.abs(got.astype(np.float64) - ring)) <= 1e-6 * np.max(np.abs(ring))
    # in place (the usual gradient all-reduce): same bits as out of place
    zs = [x.clone() for x in xs]
    ar.ar_allreduce(zs, zs, count, "f32", "sum")
    torch.cuda.synchronize()
    assert_bits_equal(to_host(zs[3], "f32"), ring, "c2 in place")


def test_c3_fsdp_reduce_scatter_then_all_gather():
    n, R = 8, 16 * MB
    xs = [workloads.device_normal(2, 0, r, n * R, 1e-2, "bf16") for r in range(n)]
    host = [to_host(x, "bf16") for x in xs]
    print("c3 rs oracle", flush=True)
    want = oracle.ring_reduce_scatter(host, "bf16", "avg")
    for sched in ("auto", "ring"):
        ys = [torch.empty(R, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
        ar.ar_reduce_scatter(xs, ys, R, "bf16", "avg", sched=sched)
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_host(ys[r], "bf16"), want[r], "c3 rs %s rank %d" % (sched, r))
    # reduce in fp32 at bf16 bytes: fp32 partials, one rounding
    print("c3 rs acc32 oracle", flush=True)
    want32 = oracle.ring_reduce_scatter(host, "bf16", "avg", acc32=True)
    ys = [torch.empty(R, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    ar.ar_reduce_scatter_ex(xs, ys, R, "bf16", "avg", acc="fp32")
    torch.cuda.synchronize()
    for r in range(n):
        assert_bits_equal(to_host(ys[r], "bf16"), want32[r], "c3 rs acc32 rank %d" % r)
    del xs
    pieces = [workloads.device_uniform(2, 1, r, R, -1.0, 1.0, "bf16") for r in range(n)]
    cat = np.concatenate([to_host(p, "bf16") for p in pieces])
    for sched in ("auto", "ring"):
        outs = [torch.empty(n * R, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
        ar.ar_all_gather(pieces, outs, R, "bf16", sched=sched)
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_host(outs[r], "bf16"), cat, "c3 ag %s rank %d" % (sched, r))
        del outs
    torch.cuda.empty_cache()


C4_OPS = ["sum", "min", "max", "avg"]


def _first_difference(got, want):
    bad = torch.nonzero(got != want)
    return int(bad[0]) if bad.numel() else -1


def _expected_int32(xs, ops, slice_elems=16 * MB):
    """The plain definition for each op (exact for int32 whatever the order),
    evaluated by the oracle on the host in slices of ``slice_elems`` elements
    per rank, each slice's result copied into a device tensor."""
    count = xs[0].numel()
    want = {op: torch.empty_like(xs[0]) for op in ops}
    for a in range(0, count, slice_elems):
        b = min(count, a + slice_elems)
        host = [to_host(x[a:b], "i32") for x in xs]
        for op in ops:
            want[op][a:b].copy_(torch.from_numpy(oracle.direct_reduce(host, "i32", op)))
    return want


@pytest.mark.parametrize("size", workloads.C4_SIZES)
def test_c4_int32_size_sweep_every_element(size):
    """n = 16 int32, 1 KB .. 1 GB per rank: every op and schedule, every
    element of every rank's output against the oracle (the oracle's result is
    computed once per op in streamed slices and compared on the device)."""
    n = workloads.C4_N
    count = size // 4
    stream = int(np.log2(size))
    xs = [workloads.device_ints(3, stream, r, count, -(1 << 20), 1 << 20, "i32") for r in range(n)]
    print("c4 oracle", size, flush=True)
    want = _expected_int32(xs, C4_OPS)
    ys = [torch.empty_like(x) for x in xs]
    for op in C4_OPS:
        for sched in ("auto", "fused", "ring", "tree", "split", "dtree"):
            print("c4", op, size, sched, flush=True)
            for y in ys:
                y.fill_(-7)
            ar.ar_allreduce(xs, ys, count, "i32", op, sched=sched)
            torch.cuda.synchronize()
            for r in range(n):
                if not torch.equal(ys[r], want[op]):
                    raise AssertionError("c4 %s %d %s rank %d: first difference at element %d"
                                         % (op, size, sched, r, _first_difference(ys[r], want[op])))
    del xs, ys, want
    torch.cuda.empty_cache()


def _c5_oracle(host, chosen):
    if chosen == "split":
        return oracle.pairwise_reduce(host, "f32", "avg")
    if chosen == "dtree":
        return oracle.dtree_allreduce(host, "f32", "avg")[0]
    if chosen == "tree":
        return oracle.tree_allreduce(host, "f32", "avg")[0]
    return oracle.ring_allreduce(host, "f32", "avg")[0]


def test_c5_bucketed_72_ranks_in_place():
    """72 ranks, all 29 buckets reduced in place back to back on one stream;
    then every bucket is checked: all 72 ranks hold the same bits (on the
    device), and rank 0's bucket equals the oracle of the planner's choice,
    evaluated on the same inputs regenerated from their seeds."""
    n = workloads.C5_N
    buckets, total = workloads.c5_buckets()
    assert len(buckets) >= 20
    count_total = total // 4
    grads = [workloads.device_spiky_normal(4, r, count_total, 1e-3, 0.01, 100.0) for r in range(n)]
    for b, (off, nbytes) in enumerate(buckets):           # back to back on one stream, in place
        a, e = off // 4, (off + nbytes) // 4
        views = [g[a:e] for g in grads]
        ar.ar_allreduce(views, views, e - a, "f32", "avg")
    torch.cuda.synchronize()
    inputs = [workloads.device_spiky_normal(4, r, count_total, 1e-3, 0.01, 100.0) for r in range(n)]
    for b, (off, nbytes) in enumerate(buckets):
        a, e = off // 4, (off + nbytes) // 4
        _same_on_all_ranks([g[a:e] for g in grads])
        chosen = ar.ar_plan("allreduce", e - a, "f32", "avg", n).chosen
        print("c5 bucket", b, nbytes, chosen, flush=True)
        want = _c5_oracle([to_host(x[a:e], "f32") for x in inputs], chosen)
        assert_bits_equal(to_host(grads[0][a:e], "f32"), want, "c5 bucket %d" % b)
    del grads, inputs
    torch.cuda.empty_cache()


def test_c5_split_one_bucket_in_place():
    """The split schedule on the 72-rank workload's first (25 MB) bucket, in place."""
    n = workloads.C5_N
    buckets, _ = workloads.c5_buckets()
    off, nbytes = buckets[0]
    count = nbytes // 4
    grads = [workloads.device_spiky_normal(4, r, count, 1e-3, 0.01, 100.0) for r in range(n)]
    host = [to_host(g, "f32") for g in grads]
    print("c5 split oracle", nbytes, flush=True)
    want = oracle.pairwise_reduce(host, "f32", "avg")
    ar.ar_allreduce(grads, grads, count, "f32", "avg", sched="split")
    torch.cuda.synchronize()
    for r in (0, 35, n - 1):
        assert_bits_equal(to_host(grads[r], "f32"), want, "c5 split rank %d" % r)
    del grads
    torch.cuda.empty_cache()


@pytest.mark.parametrize("sched", ["tree", "dtree"])
def test_c5_trees_one_bucket_in_place(sched):
    """The tree and double-tree schedules on the 72-rank workload's first
    (25 MB) bucket, in place, as a caller gets them (the streaming walk at this
    size): every element of three ranks against the oracle of the schedule."""
    n = workloads.C5_N
    buckets, _ = workloads.c5_buckets()
    off, nbytes = buckets[0]
    count = nbytes // 4
    grads = [workloads.device_spiky_normal(4, r, count, 1e-3, 0.01, 100.0) for r in range(n)]
    host = [to_host(g, "f32") for g in grads]
    print("c5 %s oracle" % sched, nbytes, flush=True)
    want = (oracle.tree_allreduce if sched == "tree" else oracle.dtree_allreduce)(host, "f32", "avg")[0]
    ar.ar_allreduce(grads, grads, count, "f32", "avg", sched=sched)
    torch.cuda.synchronize()
    for r in (0, 35, n - 1):
        assert_bits_equal(to_host(grads[r], "f32"), want, "c5 %s rank %d" % (sched, r))
    del grads, host
    torch.cuda.empty_cache()


@pytest.mark.parametrize("R", [8 << 20, (8 << 20) - 1])
def test_all_gather_past_the_cache(R):
    """16 ranks, 512 MB of pieces in all (past the 256 MB Infinity Cache, where
    the all-gather takes its streaming residency cap), whole 16-byte vectors and
    a piece length off the vector grid (the phased kernel): every output equals
    the concatenation of the pieces, bit for bit, on every rank."""
    n = 16
    xs = [workloads.device_normal(7, 3, r, R, 1.0, "f32") for r in range(n)]
    want = torch.cat(xs)
    ys = [torch.empty(n * R, device="cuda") for _ in range(n)]
    for sched in ("fused", "auto"):
        print("all-gather past the cache R=%d %s" % (R, sched), flush=True)
        for y in ys:
            y.fill_(-1.0)
        ar.ar_all_gather(xs, ys, R, "f32", sched=sched)
        torch.cuda.synchronize()
        for r in range(n):
            assert torch.equal(ys[r].view(torch.int32), want.view(torch.int32)), "%s rank %d" % (sched, r)
    del xs, ys, want
    torch.cuda.empty_cache()


BIG = (1 << 30) + (1 << 20) + 7          # fp32 elements per rank: 4.3 GB, past every 32-bit byte offset


def _windows(count, rng, k=48, w=1024):
    starts = sorted(set([0, count - w] + [int(s) for s in rng.integers(0, count - w, size=k)]))
    return [(s, s + w) for s in starts]


def _check_windows(got_t, xs_t, dtype, op, rng, count):
    """Sampled windows of an n = 2 result against the ring oracle run on the
    window (for n = 2 each element is one IEEE operation whichever rank comes
    first, so the window's own chunking gives the same bits as the call's)."""
    for lo, hi in _windows(count, rng):
        xs = [to_host(x[lo:hi], dtype) for x in xs_t]
        want = oracle.ring_allreduce(xs, dtype, op)[0]
        assert_bits_equal(to_host(got_t[lo:hi], dtype), want, "window [%d, %d)" % (lo, hi))


@pytest.mark.parametrize("sched", ["fused", "ring", "tree", "split", "dtree", "auto"])
def test_allreduce_past_4GB_per_rank(sched):
    """n = 2 fp32 all-reduce of 4.3 GB per rank (a ragged count), every
    schedule: every element equals x0 + x1 (checked on the device against
    torch's add, one IEEE addition), all ranks agree, and sampled windows
    match the oracle."""
    print("past 4 GB allreduce", sched, flush=True)
    xs = [workloads.device_normal(9, 0, r, BIG, 1.0, "f32") for r in range(2)]
    ys = [torch.empty_like(x) for x in xs]
    ar.ar_allreduce(xs, ys, BIG, "f32", "sum", sched=sched)
    torch.cuda.synchronize()
    _same_on_all_ranks(ys)
    assert torch.equal((xs[0] + xs[1]).view(torch.int32), ys[0].view(torch.int32))
    _check_windows(ys[0], xs, "f32", "sum", np.random.default_rng(1), BIG)
    del xs, ys
    torch.cuda.empty_cache()


@pytest.mark.parametrize("sched", ["fused", "ring"])
def test_reduce_scatter_and_all_gather_past_4GB(sched):
    """n = 2: reduce-scatter of 2 x 4.3 GB slices per rank, then all-gather of
    the 4.3 GB results, past every 32-bit byte offset."""
    print("past 4 GB rs/ag", sched, flush=True)
    R = BIG
    xs = [workloads.device_normal(9, 1, r, 2 * R, 1.0, "f32") for r in range(2)]
    ys = [torch.empty(R, device="cuda") for _ in range(2)]
    ar.ar_reduce_scatter(xs, ys, R, "f32", "sum", sched=sched)
    torch.cuda.synchronize()
    for c in range(2):
        assert torch.equal((xs[0][c * R:(c + 1) * R] + xs[1][c * R:(c + 1) * R]).view(torch.int32),
                           ys[c].view(torch.int32)), "slice %d" % c
    del xs
    torch.cuda.empty_cache()
    zs = [torch.empty(2 * R, device="cuda") for _ in range(2)]
    ar.ar_all_gather(ys, zs, R, "f32", sched=sched)
    torch.cuda.synchronize()
    for z in zs:
        for k in range(2):
            assert torch.equal(z[k * R:(k + 1) * R].view(torch.int32), ys[k].view(torch.int32))
    del ys, zs
    torch.cuda.empty_cache()
