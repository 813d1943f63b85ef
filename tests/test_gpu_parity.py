"""Parity of the HIP path (through the C ABI) with the CPU oracle, element by
element, at sizes the oracle finishes in seconds that still span several
tiles / LDS windows and a ragged tail.

Bar: ring and fused results are bit-identical to the ring oracle (they use
its hop order), tree results bit-identical to the tree oracle, split results
bit-identical to the pairwise oracle, double-tree results bit-identical to the
double-tree oracle; all-gather and every integer result are bit-exact by
construction."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from devutil import assert_bits_equal, empty, sync, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
ar = pytest.importorskip("reduce_scatter_amd")

DTYPES = ["f32", "bf16", "f16", "i32"]
OPS = ["sum", "prod", "min", "max", "avg"]
LANES = {"f32": 4, "i32": 4, "bf16": 8, "f16": 8}
FUSED_TILE = 64           # 16-byte vectors per fused tile (one wavefront, one per lane)


def counts_for(n, dtype):
    u = LANES[dtype]
    return [1, 5, u * n * 3, u * n * 3 + 1, n * 512 * u * 2 + u * 3 + 3]


def inputs(seed, n, count, dtype, op):
    kind = "pos" if op == "prod" else "normal"
    return [workloads.random_values(seed, n * 1000 + count, r, count, dtype, kind) for r in range(n)]


def reference(sched, xs, dtype, op):
    """The oracle of a schedule's reduction order (AUTO: of the planner's choice)."""
    if sched == "auto":
        sched = ar.ar_plan("allreduce", xs[0].size, dtype, op, len(xs)).chosen
    if sched == "tree":
        return oracle.tree_allreduce(xs, dtype, op)
    if sched == "split":
        return [oracle.pairwise_reduce(xs, dtype, op)] * len(xs)
    if sched == "dtree":
        return oracle.dtree_allreduce(xs, dtype, op)
    return oracle.ring_allreduce(xs, dtype, op)


def run_allreduce(xs, dtype, op, sched, inplace=False):
    n = len(xs)
    d_in = [to_device(x, dtype) for x in xs]
    d_out = d_in if inplace else [empty(x.size, dtype, 0) for x in xs]
    ar.ar_allreduce(d_in, d_out, xs[0].size, dtype, op, sched=sched)
    sync()
    return [to_host(t, dtype) for t in d_out]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
def test_allreduce_matches_oracle(dtype, op):
    for n in (1, 2, 3, 5, 8, 16):
        for count in counts_for(n, dtype):
            print("allreduce", dtype, op, "n=%d count=%d" % (n, count), flush=True)
            xs = inputs(1, n, count, dtype, op)
            for sched in ("fused", "ring", "tree", "split", "dtree", "auto"):
                got = run_allreduce(xs, dtype, op, sched)
                ref = reference(sched, xs, dtype, op)
                for r in range(n):
                    assert_bits_equal(got[r], ref[r], "%s %s %s n=%d count=%d rank %d" % (sched, dtype, op, n, count, r))


@pytest.mark.parametrize("dtype", DTYPES)
def test_allreduce_in_place_equals_out_of_place(dtype):
    n, count = 8, 8 * FUSED_TILE * 8 + 13
    for op in OPS:
        xs = inputs(2, n, count, dtype, op)
        for sched in ("fused", "ring", "tree", "split", "dtree"):
            a = run_allreduce(xs, dtype, op, sched)
            b = run_allreduce(xs, dtype, op, sched, inplace=True)
            for r in range(n):
                assert_bits_equal(b[r], a[r], "in place %s %s %s" % (sched, dtype, op))


@pytest.mark.parametrize("dtype", DTYPES)
def test_allreduce_element_wise_path(dtype):
    """Buffers one element past a 16-byte boundary (all at that one phase:
    the shifted-frame path) give the same results as the oracle for every
    schedule."""
    n, count = 5, 3001
    for op in ("sum", "avg", "max"):
        xs = inputs(3, n, count, dtype, op)
        for sched in ("fused", "ring", "tree", "split", "dtree"):
            d_in = [to_device(np.concatenate([x[:1], x]), dtype)[1:] for x in xs]
            d_out = [empty(count + 1, dtype, 0)[1:] for _ in xs]
            assert d_in[0].data_ptr() % 16 != 0
            ar.ar_allreduce(d_in, d_out, count, dtype, op, sched=sched)
            sync()
            ref = reference(sched, xs, dtype, op)
            for r in range(n):
                assert_bits_equal(to_host(d_out[r], dtype), ref[r], "elem %s %s %s" % (sched, dtype, op))


def run_rs(xs, dtype, op, sched, inplace=False, misalign=False):
    n = len(xs)
    R = xs[0].size // n
    if misalign:
        d_in = [to_device(np.concatenate([x[:1], x]), dtype)[1:] for x in xs]
    else:
        d_in = [to_device(x, dtype) for x in xs]
    if inplace:
        d_out = [d_in[r][r * R:(r + 1) * R] for r in range(n)]
    else:
        d_out = [empty(R, dtype, 0) for _ in range(n)]
    ar.ar_reduce_scatter(d_in, d_out, R, dtype, op, sched=sched)
    sync()
    return [to_host(t, dtype) for t in d_out]


def run_ag(xs, dtype, sched, inplace=False, misalign=False):
    n = len(xs)
    R = xs[0].size
    if inplace:
        d_out = [empty(n * R, dtype, 0) for _ in range(n)]
        for r in range(n):
            d_out[r][r * R:(r + 1) * R].copy_(to_device(xs[r], dtype))
        d_in = [d_out[r][r * R:(r + 1) * R] for r in range(n)]
    elif misalign:
        d_in = [to_device(np.concatenate([x[:1], x]), dtype)[1:] for x in xs]
        d_out = [empty(n * R + 1, dtype, 0)[1:] for _ in range(n)]
    else:
        d_in = [to_device(x, dtype) for x in xs]
        d_out = [empty(n * R, dtype, 0) for _ in range(n)]
    ar.ar_all_gather(d_in, d_out, R, dtype, sched=sched)
    sync()
    return [to_host(t, dtype) for t in d_out]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
def test_reduce_scatter_and_all_gather_match_oracle(dtype, op):
    u = LANES[dtype]
    for n in (1, 2, 3, 8, 16):
        for R in (1, 3, u, u * 37, 512 * u * 2 + u * 5):
            print("rs/ag", dtype, op, "n=%d R=%d" % (n, R), flush=True)
            xs = inputs(4, n, n * R, dtype, op)
            ref = oracle.ring_reduce_scatter(xs, dtype, op)
            for sched in ("fused", "ring", "auto"):
                for kw in ({}, {"inplace": True}, {"misalign": True}):
                    got = run_rs(xs, dtype, op, sched, **kw)
                    for r in range(n):
                        assert_bits_equal(got[r], ref[r], "rs %s %s %s n=%d R=%d %s" % (sched, dtype, op, n, R, kw))
            if op != "sum":
                continue
            pieces = [workloads.random_values(5, n, r, R, dtype) for r in range(n)]
            want = oracle.ring_all_gather(pieces, dtype)
            for sched in ("fused", "ring", "auto"):
                for kw in ({}, {"inplace": True}, {"misalign": True}):
                    got = run_ag(pieces, dtype, sched, **kw)
                    for r in range(n):
                        assert_bits_equal(got[r], want[r], "ag %s %s n=%d R=%d %s" % (sched, dtype, n, R, kw))


@pytest.mark.parametrize("dtype", DTYPES)
def test_allreduce_equals_reduce_scatter_then_all_gather(dtype):
    """all-reduce = reduce-scatter + all-gather, bit for bit (count a multiple
    of n 16-byte units, so the two calls cut the same chunks)."""
    n = 8
    u = LANES[dtype]
    R = u * 1000
    for op in OPS:
        xs = inputs(6, n, n * R, dtype, op)
        for sched in ("fused", "ring"):
            full = run_allreduce(xs, dtype, op, sched)
            parts = run_rs(xs, dtype, op, sched)
            gathered = run_ag(parts, dtype, sched)
            for r in range(n):
                assert_bits_equal(gathered[r], full[r], "AR vs RS+AG %s %s %s" % (sched, dtype, op))


def test_c1_workload_every_schedule():
    """C1: n = 4, fp32, 1024 integer-valued elements (exact sums); AR by every
    schedule, RS on the same input and AG of the RS outputs, all against the
    exact integer sum."""
    xs = workloads.c1_inputs()
    want = sum(x.astype(np.int64) for x in xs).astype(np.float32)
    for sched in ("fused", "ring", "tree", "split", "dtree", "auto"):
        for y in run_allreduce(xs, "f32", "sum", sched):
            assert_bits_equal(y, want, "c1 " + sched)
    parts = run_rs(xs, "f32", "sum", "auto")
    for r in range(4):
        assert_bits_equal(parts[r], want[r * 256:(r + 1) * 256], "c1 rs")
    for y in run_ag(parts, "f32", "auto"):
        assert_bits_equal(y, want, "c1 ag")


def test_large_rank_counts():
    """n up to the table limit (128) and the bucketed workload's 72."""
    for n in (72, 128):
        count = n * 4 * 40 + 3
        xs = inputs(7, n, count, "f32", "avg")
        for sched in ("fused", "ring", "tree", "split", "dtree"):
            got = run_allreduce(xs, "f32", "avg", sched)
            ref = reference(sched, xs, "f32", "avg")
            for r in (0, n // 2, n - 1):
                assert_bits_equal(got[r], ref[r], "n=%d %s" % (n, sched))


@pytest.mark.parametrize("dtype", DTYPES)
def test_split_many_ranks_every_op(dtype):
    """The split schedule at rank counts that exercise every ranks-per-wave
    choice (1, 2, 4, 8 ranks per wave; partial last waves), all ops."""
    u = LANES[dtype]
    for n in (17, 31, 33, 72, 100, 128):
        count = 64 * u * 3 + u * 5 + 3                   # 3 full tiles, a partial tile, a ragged tail
        for op in OPS:
            print("split", dtype, op, "n=%d" % n, flush=True)
            xs = inputs(8, n, count, dtype, op)
            want = oracle.pairwise_reduce(xs, dtype, op)
            got = run_allreduce(xs, dtype, op, "split")
            for r in (0, n // 2, n - 1):
                assert_bits_equal(got[r], want, "split %s %s n=%d rank %d" % (dtype, op, n, r))
            if dtype == "i32" or op in ("min", "max"):
                assert_bits_equal(want, oracle.direct_reduce(xs, dtype, op), "split exact")


@pytest.mark.parametrize("layout", ["default", "0", "1"])
def test_reduce_scatter_many_ranks_both_layouts(layout, monkeypatch):
    """Aligned reduce-scatter past 16 ranks through the any-n fused kernel
    (AR_RS_PHASED=0), the phased kernel's layout (1) and the default choice
    between them: every dtype, rank counts on both sides of the choice, whole
    tiles and a partial one, fused and ring schedules, bit for bit against
    the oracle."""
    if layout != "default":
        monkeypatch.setenv("AR_RS_PHASED", layout)
    for dtype in DTYPES:
        u = LANES[dtype]
        R = 64 * u * 3 + u
        for n in (17, 20, 24, 33, 40, 72, 128):
            op = OPS[(n + u) % len(OPS)]
            print("rs many ranks", layout, dtype, op, "n=%d R=%d" % (n, R), flush=True)
            xs = inputs(170 + n, n, n * R, dtype, op)
            ref = oracle.ring_reduce_scatter(xs, dtype, op)
            for sched in ("fused",) if n in (40, 128) else ("fused", "ring"):
                got = run_rs(xs, dtype, op, sched)
                for r in range(n):
                    assert_bits_equal(got[r], ref[r], "rs %s %s %s n=%d rank %d" % (layout, dtype, op, n, r))


@pytest.mark.parametrize("halves", ["default", "0"])
def test_allreduce_many_ranks_halves(halves, monkeypatch):
    """The fused all-reduce past 16 ranks as reduce-scatter half then
    all-gather half over the all-reduce's own chunks (the default), and as the
    wide one-pass kernel (AR_AR_HALVES=0): every dtype, ragged counts (chunks
    of unequal length, a partial last vector), in and out of place, bit for
    bit against the ring oracle, every rank checked."""
    if halves != "default":
        monkeypatch.setenv("AR_AR_HALVES", halves)
    for dtype in DTYPES:
        u = LANES[dtype]
        for n in (17, 24, 33, 72, 128):
            count = 64 * u * 2 * n + u * (n // 3) + 5
            op = OPS[(n + u) % len(OPS)]
            print("ar halves", halves, dtype, op, "n=%d count=%d" % (n, count), flush=True)
            xs = inputs(190 + n, n, count, dtype, op)
            ref = oracle.ring_allreduce(xs, dtype, op)
            got = run_allreduce(xs, dtype, op, "fused")
            for r in range(n):
                assert_bits_equal(got[r], ref[r], "ar %s %s %s n=%d rank %d" % (halves, dtype, op, n, r))
            got = run_allreduce(xs, dtype, op, "fused", inplace=True)
            for r in (0, n // 2, n - 1):
                assert_bits_equal(got[r], ref[r], "ar in place %s %s %s n=%d rank %d" % (halves, dtype, op, n, r))


@pytest.mark.parametrize("halves", ["default", "0"])
def test_fused_many_ranks_tiny_counts(halves, monkeypatch):
    """The fused all-reduce and reduce-scatter past 16 ranks at counts where
    most chunks hold no vector or one (fewer vectors than ranks, a partial last
    vector, a count below one vector), both all-reduce paths, against the
    oracle bit for bit."""
    if halves != "default":
        monkeypatch.setenv("AR_AR_HALVES", halves)
        monkeypatch.setenv("AR_RS_PHASED", "0")
    for dtype in ("f32", "bf16"):
        u = LANES[dtype]
        for n in (17, 72, 128):
            for count in sorted({1, 3, u + 1, u * (n // 2) + 1, u * n - 1, u * n + 1, u * (n + 1)}):
                op = OPS[(n + count) % len(OPS)]
                xs = inputs(210 + count % 97, n, count, dtype, op)
                ref = oracle.ring_allreduce(xs, dtype, op)
                got = run_allreduce(xs, dtype, op, "fused")
                for r in (0, n // 2, n - 1):
                    assert_bits_equal(got[r], ref[r], "ar tiny %s %s %s n=%d count=%d rank %d" % (
                        halves, dtype, op, n, count, r))
            for R in (u, 2 * u):
                xs = inputs(220 + R, n, n * R, dtype, "sum")
                ref = oracle.ring_reduce_scatter(xs, dtype, "sum")
                got = run_rs(xs, dtype, "sum", "fused")
                for r in range(n):
                    assert_bits_equal(got[r], ref[r], "rs tiny %s %s n=%d R=%d rank %d" % (halves, dtype, n, R, r))


def _at_offset(x, dtype, off_bytes):
    """A device copy of host array x starting off_bytes past a fresh allocation."""
    pad = off_bytes // (4 if dtype in ("f32", "i32") else 2)
    return to_device(np.concatenate([np.zeros(pad, x.dtype), x]), dtype)[pad:]


def _empty_at_offset(count, dtype, off_bytes):
    pad = off_bytes // (4 if dtype in ("f32", "i32") else 2)
    return empty(count + pad, dtype, 0)[pad:]


OFFSET_SETS = {
    "same 48 B": lambda n: [48] * n,
    "same 1040 B": lambda n: [1040] * n,
    "mixed": lambda n: [16 * (r % 7) for r in range(n)],
}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiles_cut_on_an_aligned_grid(dtype):
    """Rank buffers 16-byte aligned but off 1 KB boundaries (the same offset on
    every rank, or different ones): the fused and split kernels cut tiles on
    rank 0's aligned grid, leaving partial first tiles; results unchanged."""
    u = LANES[dtype]
    for n in (3, 8, 72):
        count = 64 * u * 5 + u * 3 + 1
        for label, offs in OFFSET_SETS.items():
            offsets = offs(n)
            print("aligned grid", dtype, n, label, flush=True)
            xs = inputs(9, n, count, dtype, "avg")
            for sched in ("fused", "split", "ring", "tree", "dtree"):
                d_in = [_at_offset(x, dtype, o) for x, o in zip(xs, offsets)]
                d_out = [_empty_at_offset(count, dtype, (o + 32) % 1024) for o in offsets]
                ar.ar_allreduce(d_in, d_out, count, dtype, "avg", sched=sched)
                ar.ar_allreduce(d_in, d_in, count, dtype, "avg", sched=sched)          # in place
                sync()
                ref = reference(sched, xs, dtype, "avg")
                for r in (0, n // 2, n - 1):
                    assert_bits_equal(to_host(d_out[r], dtype), ref[r], "%s n=%d %s rank %d" % (sched, n, label, r))
                    assert_bits_equal(to_host(d_in[r], dtype), ref[r], "%s n=%d %s in place" % (sched, n, label))
            R = 64 * u * 3 + u * 2                                  # 16-byte multiple: the vector path
            ys = inputs(10, n, n * R, dtype, "sum")
            want = oracle.ring_reduce_scatter(ys, dtype, "sum")
            pieces = [workloads.random_values(11, n, r, R, dtype) for r in range(n)]
            gathered = oracle.ring_all_gather(pieces, dtype)
            for sched in ("fused", "ring"):
                d_in = [_at_offset(y, dtype, o) for y, o in zip(ys, offsets)]
                d_out = [_empty_at_offset(R, dtype, (o + 16) % 1024) for o in offsets]
                ar.ar_reduce_scatter(d_in, d_out, R, dtype, "sum", sched=sched)
                g_in = [_at_offset(pc, dtype, o) for pc, o in zip(pieces, offsets)]
                g_out = [_empty_at_offset(n * R, dtype, (o + 80) % 1024) for o in offsets]
                ar.ar_all_gather(g_in, g_out, R, dtype, sched=sched)
                sync()
                for r in (0, n // 2, n - 1):
                    assert_bits_equal(to_host(d_out[r], dtype), want[r], "rs %s n=%d %s" % (sched, n, label))
                    assert_bits_equal(to_host(g_out[r], dtype), gathered[r], "ag %s n=%d %s" % (sched, n, label))


WIDE_CASES = [("f32", "avg"), ("bf16", "sum"), ("f16", "avg"), ("i32", "avg"), ("f32", "max")]


@pytest.mark.parametrize("dtype,op", WIDE_CASES)
def test_wide_fused_whole_shared_and_edge_tiles(dtype, op):
    """Past 16 ranks the fused all-reduce cuts the chunks on a grid of 64*U
    vector tiles (U = 16 for 4-byte types, 8 for 2-byte ones): whole tiles
    inside a chunk, shared tiles across a chunk boundary (one workgroup walks
    both chunks' hop orders), and partial tiles at the buffer ends or where a
    tile holds three or more chunks.  Chunks of several tiles, of 1.5 tiles
    and of a third of a tile; the grid shifted by the buffers' offset; every
    buffer at one 16-byte phase (the shifted frame, whose vector across each
    chunk boundary goes to the element-wise kernel); every element of every
    rank, in place and out of place."""
    u = LANES[dtype]
    e = 4 if u == 4 else 2
    tile_elems = 64 * (16 if u == 4 else 8) * u
    layouts = (("aligned", lambda n: [0] * n), ("off the tile grid", lambda n: [48] * n),
               ("mixed", lambda n: [16 * (r % 7) for r in range(n)]), ("one phase", lambda n: [48 + e] * n))
    for n in (17, 72):
        for count in (n * (3 * tile_elems + 1000) + 7, n * (3 * tile_elems // 2) + 13, n * (tile_elems // 3) + 5):
            xs = inputs(31, n, count, dtype, op)
            ref = oracle.ring_allreduce(xs, dtype, op)
            for label, offs in layouts:
                offsets = offs(n)
                print("wide fused", dtype, op, n, count, label, flush=True)
                d_in = [_at_offset(x, dtype, o) for x, o in zip(xs, offsets)]
                d_out = [_empty_at_offset(count, dtype, (o + 32) % 1024) for o in offsets]
                ar.ar_allreduce(d_in, d_out, count, dtype, op, sched="fused")
                ar.ar_allreduce(d_in, d_in, count, dtype, op, sched="fused")          # in place
                sync()
                for r in range(n):
                    assert_bits_equal(to_host(d_out[r], dtype), ref[r], "n=%d %d %s rank %d" % (n, count, label, r))
                    assert_bits_equal(to_host(d_in[r], dtype), ref[r], "n=%d %d %s rank %d in place" % (n, count, label, r))
                del d_in, d_out


NUMERICS = [("storage", "split"), ("fp32", "prescale"), ("fp32", "split")]


def _numerics_reference(sched, xs, dtype, op, acc, avg, coll="allreduce"):
    kw = {"acc32": acc == "fp32", "avg_split": avg == "split"}
    if coll == "reduce_scatter":
        return oracle.ring_reduce_scatter(xs, dtype, op, **kw)
    if sched == "tree":
        return oracle.tree_allreduce(xs, dtype, op, **kw)
    if sched == "dtree":
        return oracle.dtree_allreduce(xs, dtype, op, **kw)
    if sched == "split":
        return [oracle.pairwise_reduce(xs, dtype, op, **kw)] * len(xs)
    return oracle.ring_allreduce(xs, dtype, op, **kw)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16", "i32"])
def test_numerics_variants_match_oracle(dtype):
    """fp32 partials (fused; other schedules refuse bf16 / fp16) and the split
    avg divisor (every schedule), all-reduce and reduce-scatter, against the
    oracle with the same options; vector and element-wise paths."""
    u = LANES[dtype]
    for n in (3, 8, 16, 72):
        count = 64 * u * 4 + u * 3 + 5
        for op in ("sum", "avg", "prod", "max"):
            xs = inputs(20, n, count, dtype, op)
            for acc, avg in NUMERICS:
                refuse = acc == "fp32" and dtype in ("bf16", "f16")
                for sched in ("fused", "ring", "tree", "split", "dtree", "auto"):
                    print("numerics", dtype, op, n, acc, avg, sched, flush=True)
                    d_in = [to_device(x, dtype) for x in xs]
                    d_out = [empty(count, dtype, 0) for _ in xs]
                    if refuse and sched not in ("fused", "auto"):
                        with pytest.raises(ar.ArError):
                            ar.ar_allreduce_ex(d_in, d_out, count, dtype, op, sched=sched, acc=acc, avg=avg)
                        continue
                    ar.ar_allreduce_ex(d_in, d_out, count, dtype, op, sched=sched, acc=acc, avg=avg)
                    sync()
                    used = sched
                    if sched == "auto":
                        used = "fused" if refuse else ar.ar_plan("allreduce", count, dtype, op, n).chosen
                    ref = _numerics_reference(used, xs, dtype, op, acc, avg)
                    for r in (0, n - 1):
                        assert_bits_equal(to_host(d_out[r], dtype), ref[r], "%s %s %s n=%d %s/%s rank %d" % (
                            sched, dtype, op, n, acc, avg, r))
                # element-wise path (buffers off 16-byte alignment), fused
                d_in = [to_device(np.concatenate([x[:1], x]), dtype)[1:] for x in xs]
                d_out = [empty(count + 1, dtype, 0)[1:] for _ in xs]
                ar.ar_allreduce_ex(d_in, d_out, count, dtype, op, sched="fused", acc=acc, avg=avg)
                sync()
                ref = _numerics_reference("fused", xs, dtype, op, acc, avg)
                assert_bits_equal(to_host(d_out[0], dtype), ref[0], "elem %s %s n=%d %s/%s" % (dtype, op, n, acc, avg))
            # reduce-scatter
            R = 64 * u * 2 + u
            ys = inputs(21, n, n * R, dtype, op)
            for acc, avg in NUMERICS:
                ref = _numerics_reference("ring", ys, dtype, op, acc, avg, coll="reduce_scatter")
                for sched in ("fused", "ring"):
                    if acc == "fp32" and dtype in ("bf16", "f16") and sched == "ring":
                        continue
                    d_in = [to_device(y, dtype) for y in ys]
                    d_out = [empty(R, dtype, 0) for _ in ys]
                    ar.ar_reduce_scatter_ex(d_in, d_out, R, dtype, op, sched=sched, acc=acc, avg=avg)
                    sync()
                    for r in (0, n - 1):
                        assert_bits_equal(to_host(d_out[r], dtype), ref[r], "rs %s %s %s n=%d %s/%s" % (
                            sched, dtype, op, n, acc, avg))


def _at_phase(x, dtype, k, extra=0):
    """A device copy of ``x`` starting ``k`` elements past a 16-byte boundary
    (``extra`` more elements of room after it)."""
    d = to_device(np.concatenate([np.zeros(k, dtype=x.dtype), x, np.zeros(extra, dtype=x.dtype)]), dtype)
    assert d.data_ptr() % 16 == 0
    return d[k:k + x.size]


@pytest.mark.parametrize("dtype", DTYPES)
def test_allreduce_buffers_at_one_phase(dtype):
    """Buffers that all sit at the same 16-byte phase (element-aligned, not
    16-byte aligned): the vectors run from the first 16-byte boundary and the
    element-wise kernels take each chunk's head, the vector across each chunk
    boundary and the tail.  Every phase, every schedule, n from 2 to 72
    (chunks of zero, one and many vectors), in and out of place, against the
    oracle bit for bit; pointers at two different phases go element-wise."""
    u = LANES[dtype]
    for n in (2, 3, 8, 16, 17, 72):
        for count in sorted({u - 1, 3 * u + 1, n * u, n * u * 2 + 3, 64 * u * 3 + u * n + 5}):
            for k in range(1, u):
                op = ("sum", "avg", "prod", "max")[(n + k) % 4]
                xs = inputs(80 + k, n, count, dtype, op)
                print("phase", dtype, op, "n=%d count=%d k=%d" % (n, count, k), flush=True)
                for sched in ("fused", "ring", "tree", "dtree", "split"):
                    ref = reference(sched, xs, dtype, op)
                    d_in = [_at_phase(x, dtype, k) for x in xs]
                    d_out = [_at_phase(np.zeros_like(x), dtype, k) for x in xs]
                    ar.ar_allreduce(d_in, d_out, count, dtype, op, sched=sched)
                    sync()
                    for r in (0, n // 2, n - 1):
                        assert_bits_equal(to_host(d_out[r], dtype), ref[r], "phase %s %s %s n=%d count=%d k=%d rank %d"
                                          % (sched, dtype, op, n, count, k, r))
                    ar.ar_allreduce(d_in, d_in, count, dtype, op, sched=sched)          # in place
                    sync()
                    for r in (0, n - 1):
                        assert_bits_equal(to_host(d_in[r], dtype), ref[r], "phase in place %s %s %s n=%d count=%d k=%d"
                                          % (sched, dtype, op, n, count, k))
    # sends and receives at different phases: the element-wise path, same bits
    n, count = 8, 64 * u * 2 + 7
    xs = inputs(90, n, count, dtype, "sum")
    d_in = [_at_phase(x, dtype, 1) for x in xs]
    d_out = [_at_phase(np.zeros_like(x), dtype, u - 1) for x in xs]
    ar.ar_allreduce(d_in, d_out, count, dtype, "sum", sched="fused")
    sync()
    ref = reference("fused", xs, dtype, "sum")
    for r in range(n):
        assert_bits_equal(to_host(d_out[r], dtype), ref[r], "mixed phases rank %d" % r)


@pytest.mark.parametrize("dtype", DTYPES)
def test_allreduce_mixed_phases_dword_aligned(dtype, monkeypatch):
    """Every rank's buffers at its own 16-byte phase, each a multiple of 4
    bytes (in and out of place): the fused kernels run on the callers'
    dword-aligned pointers in ring order, the element-wise kernel takes the
    count mod lanes tail.  n from 2 to 72 (the wide kernel past 16 ranks, chunk boundaries
    inside tiles), counts of less than one vector to several tiles per chunk
    with ragged tails, every op, the fused and ring schedules, bit for bit
    against the oracle and against the element-wise path."""
    u = LANES[dtype]
    w = u // 4                                          # elements per 4-byte word
    for n in (2, 3, 8, 16, 17, 72):
        for count in sorted({3, u * n + 1, 64 * u * 3 + u * n + 5, 64 * 8 * u * 3 + u * n + 7}):
            op = OPS[(n + count) % len(OPS)]
            xs = inputs(110 + n, n, count, dtype, op)
            ref = oracle.ring_allreduce(xs, dtype, op)
            print("dword phases", dtype, op, "n=%d count=%d" % (n, count), flush=True)
            for sched in ("fused", "ring"):
                d_in = [_at_phase(x, dtype, w * (r % 4)) for r, x in enumerate(xs)]
                d_out = [_at_phase(np.zeros_like(x), dtype, w * ((3 * r + 1) % 4)) for r, x in enumerate(xs)]
                ar.ar_allreduce(d_in, d_out, count, dtype, op, sched=sched)
                sync()
                for r in range(n):
                    assert_bits_equal(to_host(d_out[r], dtype), ref[r], "dword %s %s %s n=%d count=%d rank %d" % (
                        sched, dtype, op, n, count, r))
                ar.ar_allreduce(d_in, d_in, count, dtype, op, sched=sched)              # in place
                sync()
                for r in (0, n // 2, n - 1):
                    assert_bits_equal(to_host(d_in[r], dtype), ref[r], "dword in place %s %s %s n=%d count=%d rank %d"
                                      % (sched, dtype, op, n, count, r))
    # the element-wise path gives the same bits
    n, count = 8, 64 * u * 5 + 3
    xs = inputs(119, n, count, dtype, "avg")
    outs = []
    for flag in ("1", "0"):
        monkeypatch.setenv("AR_DWORD_VECTORS", flag)
        d_in = [_at_phase(x, dtype, w * (r % 4)) for r, x in enumerate(xs)]
        d_out = [_at_phase(np.zeros_like(x), dtype, w * ((r + 2) % 4)) for r, x in enumerate(xs)]
        ar.ar_allreduce(d_in, d_out, count, dtype, "avg", sched="fused")
        sync()
        outs.append([to_host(d, dtype) for d in d_out])
    for r in range(n):
        assert_bits_equal(outs[0][r], outs[1][r], "dword against element-wise rank %d" % r)


@pytest.mark.parametrize("dtype", DTYPES)
def test_reduce_scatter_mixed_phases_dword_aligned(dtype, monkeypatch):
    """Reduce-scatter with every rank's input and output at its own 16-byte
    phase, each a multiple of 4 bytes: the phased kernel's word-aligned loads
    on the callers' pointers (2-byte slices of an odd length shift by half a
    word), the element-wise kernel each slice's last R mod lanes elements.
    n from 2 to 24 (compile-time and any-n kernels), slices shorter than a
    vector up to several tiles, every op, fused and ring, out of place and in
    place, bit for bit against the oracle and against the element-wise
    path."""
    u = LANES[dtype]
    w = u // 4                                          # elements per 4-byte word
    for n in (2, 3, 8, 16, 17, 24):
        for R in sorted({3, u * 5 + 1, 64 * u * 2 * 3 + 2, 64 * u * 7 + u, 64 * u * 2 * 5 + 1}):
            op = OPS[(n + R) % len(OPS)]
            xs = inputs(130 + n, n, n * R, dtype, op)
            ref = oracle.ring_reduce_scatter(xs, dtype, op)
            print("dword rs phases", dtype, op, "n=%d R=%d" % (n, R), flush=True)
            for sched in ("fused", "ring"):
                d_in = [_at_phase(x, dtype, w * (r % 4)) for r, x in enumerate(xs)]
                d_out = [_at_phase(np.zeros(R, dtype=xs[0].dtype), dtype, w * ((r + 1) % 4)) for r in range(n)]
                ar.ar_reduce_scatter(d_in, d_out, R, dtype, op, sched=sched)
                sync()
                for r in range(n):
                    assert_bits_equal(to_host(d_out[r], dtype), ref[r], "dword rs %s %s %s n=%d R=%d rank %d" % (
                        sched, dtype, op, n, R, r))
                d_in = [_at_phase(x, dtype, w * ((2 * r + 1) % 4)) for r, x in enumerate(xs)]
                ar.ar_reduce_scatter(d_in, [d_in[r][r * R:(r + 1) * R] for r in range(n)], R, dtype, op, sched=sched)
                sync()
                for r in (0, n // 2, n - 1):
                    assert_bits_equal(to_host(d_in[r][r * R:(r + 1) * R], dtype), ref[r],
                                      "dword rs in place %s %s %s n=%d R=%d rank %d" % (sched, dtype, op, n, R, r))
    n, R = 8, 64 * u * 3 + 1
    xs = inputs(139, n, n * R, dtype, "avg")
    outs = []
    for flag in ("1", "0"):
        monkeypatch.setenv("AR_DWORD_VECTORS", flag)
        d_in = [_at_phase(x, dtype, w * (r % 4)) for r, x in enumerate(xs)]
        d_out = [_at_phase(np.zeros(R, dtype=xs[0].dtype), dtype, w * ((r + 3) % 4)) for r in range(n)]
        ar.ar_reduce_scatter(d_in, d_out, R, dtype, "avg", sched="fused")
        sync()
        outs.append([to_host(d, dtype) for d in d_out])
    for r in range(n):
        assert_bits_equal(outs[0][r], outs[1][r], "dword rs against element-wise rank %d" % r)


@pytest.mark.parametrize("dtype", DTYPES)
def test_all_gather_mixed_phases_dword_aligned(dtype, monkeypatch):
    """All-gather with every rank's input and output at its own 16-byte phase,
    pointers and piece length whole 4-byte words: the phased kernel on the
    callers' pointers with one word-aligned load per vector, the element-wise
    kernel each piece's ends.  n from 2 to 24, pieces shorter than a vector up
    to several tiles, out of place and in place, bit for bit against the
    oracle and against the element-wise path."""
    u = LANES[dtype]
    w = u // 4                                          # elements per 4-byte word
    for n in (2, 3, 8, 16, 17, 24):
        for R in sorted({2, u * 5 + 2, 64 * u * 2 * 3 + 2, 64 * u * 7 + u}):
            R = R - R % w if w > 1 else R               # whole words
            pieces = inputs(150 + n, n, R, dtype, "sum")
            want = oracle.ring_all_gather(pieces, dtype)
            print("dword ag phases", dtype, "n=%d R=%d" % (n, R), flush=True)
            for sched in ("fused", "ring"):
                g_in = [_at_phase(x, dtype, w * (r % 4)) for r, x in enumerate(pieces)]
                g_out = [_at_phase(np.zeros(n * R, dtype=pieces[0].dtype), dtype, w * ((3 * r + 2) % 4)) for r in range(n)]
                ar.ar_all_gather(g_in, g_out, R, dtype, sched=sched)
                sync()
                for r in range(n):
                    assert_bits_equal(to_host(g_out[r], dtype), want[r], "dword ag %s %s n=%d R=%d rank %d" % (
                        sched, dtype, n, R, r))
                # in place: rank r's piece already sits at its own place in its output
                g_full = [_at_phase(np.concatenate(pieces), dtype, w * ((r + 1) % 4)) for r in range(n)]
                ar.ar_all_gather([g_full[r][r * R:(r + 1) * R] for r in range(n)], g_full, R, dtype, sched=sched)
                sync()
                for r in (0, n // 2, n - 1):
                    assert_bits_equal(to_host(g_full[r], dtype), want[r], "dword ag in place %s %s n=%d R=%d rank %d"
                                      % (sched, dtype, n, R, r))
    n, R = 8, 64 * u * 3 + 2 * w
    pieces = inputs(159, n, R, dtype, "sum")
    outs = []
    for flag in ("1", "0"):
        monkeypatch.setenv("AR_DWORD_VECTORS", flag)
        g_in = [_at_phase(x, dtype, w * (r % 4)) for r, x in enumerate(pieces)]
        g_out = [_at_phase(np.zeros(n * R, dtype=pieces[0].dtype), dtype, w * ((r + 3) % 4)) for r in range(n)]
        ar.ar_all_gather(g_in, g_out, R, dtype, sched="fused")
        sync()
        outs.append([to_host(d, dtype) for d in g_out])
    for r in range(n):
        assert_bits_equal(outs[0][r], outs[1][r], "dword ag against element-wise rank %d" % r)


@pytest.mark.parametrize("dtype", DTYPES)
def test_reduce_scatter_and_all_gather_at_phases(dtype):
    """Inputs at one 16-byte phase and outputs at another (every pair of
    element offsets within a vector): the phased pass writes the output frame
    from the outputs' first 16-byte boundary, the element-wise kernels the
    rest; slices of whole and partial vectors, n = 2, 3, 8 and 17, against the
    oracle bit for bit.  Inputs at mixed phases go element-wise."""
    u = LANES[dtype]
    pairs = [(ks, kr) for ks in range(u) for kr in range(u)]
    for n in (2, 3, 8, 17):
        for R in (1, u - 1, u * 5, 64 * u + 3, 64 * u * 2):
            for ks, kr in pairs[(n + R) % 3::3]:
                op = OPS[(ks + kr + n) % len(OPS)]
                print("rs/ag phases", dtype, op, "n=%d R=%d ks=%d kr=%d" % (n, R, ks, kr), flush=True)
                xs = inputs(95 + ks, n, n * R, dtype, op)
                ref = oracle.ring_reduce_scatter(xs, dtype, op)
                d_in = [_at_phase(x, dtype, ks) for x in xs]
                d_out = [_at_phase(np.zeros(R, dtype=xs[0].dtype), dtype, kr) for _ in range(n)]
                ar.ar_reduce_scatter(d_in, d_out, R, dtype, op, sched="fused")
                sync()
                for r in range(n):
                    assert_bits_equal(to_host(d_out[r], dtype), ref[r], "rs %s %s n=%d R=%d ks=%d kr=%d rank %d" % (
                        dtype, op, n, R, ks, kr, r))
                pieces = inputs(96 + kr, n, R, dtype, "sum")
                want = oracle.ring_all_gather(pieces, dtype)
                g_in = [_at_phase(x, dtype, ks) for x in pieces]
                g_out = [_at_phase(np.zeros(n * R, dtype=xs[0].dtype), dtype, kr) for _ in range(n)]
                ar.ar_all_gather(g_in, g_out, R, dtype, sched="fused")
                sync()
                for r in (0, n - 1):
                    assert_bits_equal(to_host(g_out[r], dtype), want[r], "ag %s n=%d R=%d ks=%d kr=%d rank %d" % (
                        dtype, n, R, ks, kr, r))
    # inputs at mixed phases: element-wise
    n, R = 8, 64 * u + 3
    xs = inputs(97, n, n * R, dtype, "sum")
    d_in = [_at_phase(x, dtype, r % u) for r, x in enumerate(xs)]
    d_out = [_at_phase(np.zeros(R, dtype=xs[0].dtype), dtype, 1) for _ in range(n)]
    ar.ar_reduce_scatter(d_in, d_out, R, dtype, "sum", sched="fused")
    sync()
    ref = oracle.ring_reduce_scatter(xs, dtype, "sum")
    for r in range(n):
        assert_bits_equal(to_host(d_out[r], dtype), ref[r], "rs mixed phases rank %d" % r)


@pytest.mark.parametrize("form", ["funnel", "hybrid", "words"])
def test_phased_reduce_scatter_load_forms(form, monkeypatch):
    """The phased reduce-scatter's two ways of reading a lane's 16 input bytes
    (an aligned pair and a funnel shift, or one load from the word boundary
    below them with a byte shift where the phase is not whole words), forced
    one at a time and mixed per slice: n = 2, 5, 8 and 16 (compile-time
    kernels, whole and partial tiles, the input's last tiles) and 17 (any n),
    bf16 / fp16 / fp32 with odd slice lengths, every op, bit for bit against
    the oracle."""
    monkeypatch.setenv("AR_PHASED_FORM", form)
    for dtype in ("bf16", "f16", "f32"):
        u = LANES[dtype]
        for n in (2, 5, 8, 16, 17):
            for R in (64 * u * 2 * 5 + 1, 64 * u * 3 - 1):
                op = OPS[(n + R) % len(OPS)]
                print("phased form", form, dtype, op, "n=%d R=%d" % (n, R), flush=True)
                xs = inputs(40 + n, n, n * R, dtype, op)
                ref = oracle.ring_reduce_scatter(xs, dtype, op)
                got = run_rs(xs, dtype, op, "fused")
                for r in range(n):
                    assert_bits_equal(got[r], ref[r], "rs %s %s %s n=%d R=%d rank %d" % (form, dtype, op, n, R, r))


@pytest.mark.parametrize("dtype", DTYPES)
def test_slices_off_the_vector_grid(dtype):
    """Slices whose byte length is not a multiple of 16 bytes, with 16-byte
    aligned buffers (the phased pass for every whole output vector, the
    element-wise kernels for the ends): every residue of the slice length
    modulo a vector, slices shorter than one vector, n from 2 to 17 (17 takes
    the any-n kernels), every op, fp32 partials and the split avg divisor,
    reduce-scatter and all-gather, bit for bit against the oracle."""
    u = LANES[dtype]
    sizes = [u - 1, u + 1] + [64 * u * 2 + j for j in range(1, u)]
    for n in (2, 3, 5, 8, 16, 17):
        for R in sizes:
            print("phased", dtype, "n=%d R=%d" % (n, R), flush=True)
            for op in OPS:
                xs = inputs(50 + R, n, n * R, dtype, op)
                ref = oracle.ring_reduce_scatter(xs, dtype, op)
                for sched in ("fused", "ring"):
                    got = run_rs(xs, dtype, op, sched)
                    for r in range(n):
                        assert_bits_equal(got[r], ref[r], "rs %s %s %s n=%d R=%d rank %d" % (
                            sched, dtype, op, n, R, r))
            pieces = inputs(60 + R, n, R, dtype, "sum")
            want = oracle.ring_all_gather(pieces, dtype)
            for sched in ("fused", "ring"):
                got = run_ag(pieces, dtype, sched)
                for r in range(n):
                    assert_bits_equal(got[r], want[r], "ag %s %s n=%d R=%d rank %d" % (sched, dtype, n, R, r))
    R = 64 * u * 3 + u - 1
    for n in (3, 8, 17):
        for op in ("sum", "avg", "prod", "max"):
            ys = inputs(70, n, n * R, dtype, op)
            for acc, avg in NUMERICS:
                print("phased numerics", dtype, op, n, acc, avg, flush=True)
                ref = _numerics_reference("ring", ys, dtype, op, acc, avg, coll="reduce_scatter")
                d_in = [to_device(y, dtype) for y in ys]
                d_out = [empty(R, dtype, 0) for _ in ys]
                ar.ar_reduce_scatter_ex(d_in, d_out, R, dtype, op, sched="fused", acc=acc, avg=avg)
                sync()
                for r in range(n):
                    assert_bits_equal(to_host(d_out[r], dtype), ref[r], "rs %s %s n=%d %s/%s rank %d" % (
                        dtype, op, n, acc, avg, r))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_float_extremes_match_oracle(dtype):
    """Subnormal-range contributions (the rounding of partials and of the
    avg pre-scale among subnormals), sums and products that overflow to +inf,
    and ±0 from underflowing products, on every schedule and with both
    numerics options: the storage-type conversions keep subnormals and round
    to nearest even like the oracle's."""
    u = LANES[dtype]
    for n in (3, 8):
        count = 64 * u * 3 + 7
        xs = [workloads.random_values(30, n, r, count, dtype, "extremes") for r in range(n)]
        for op in OPS:
            for sched in ("fused", "ring", "tree", "split", "dtree"):
                print("extremes", dtype, op, n, sched, flush=True)
                got = run_allreduce(xs, dtype, op, sched)
                ref = reference(sched, xs, dtype, op)
                for r in (0, n - 1):
                    assert_bits_equal(got[r], ref[r], "extremes %s %s %s n=%d rank %d" % (sched, dtype, op, n, r))
            for acc, avg in NUMERICS:
                sched = "fused" if acc == "fp32" else "ring"
                print("extremes", dtype, op, n, acc, avg, sched, flush=True)
                d_in = [to_device(x, dtype) for x in xs]
                d_out = [empty(count, dtype, 0) for _ in xs]
                ar.ar_allreduce_ex(d_in, d_out, count, dtype, op, sched=sched, acc=acc, avg=avg)
                sync()
                ref = _numerics_reference(sched, xs, dtype, op, acc, avg)
                assert_bits_equal(to_host(d_out[0], dtype), ref[0], "extremes %s %s n=%d %s/%s" % (
                    dtype, op, n, acc, avg))


def test_one_hip_runtime_whatever_the_import_order():
    """Importing the binding before torch must not leave two HIP runtimes in
    the process (torch ships its own copy of libamdhip64); the call must work."""
    import subprocess
    import sys
    code = r'''
import reduce_scatter_amd as ar
import torch
xs = [torch.full((1000,), float(r + 1), device="cuda") for r in range(4)]
ys = [torch.empty_like(x) for x in xs]
ar.ar_allreduce(xs, ys, 1000, "f32", "sum")
torch.cuda.synchronize()
assert all(float(y.min()) == 10.0 == float(y.max()) for y in ys)
maps = open("/proc/self/maps").read()
hips = sorted({line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line})
assert len(hips) == 1, hips
print("ok", hips[0])
'''
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=100)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("sched", ["fused", "ring"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_rank_count_up_to_17(dtype, sched):
    """Every n up to 16 has its own compile-time fused and ring kernels (17
    takes the any-n paths): all-reduce, reduce-scatter and all-gather against
    the oracle, with slices on and off the 16-byte grid."""
    u = LANES[dtype]
    for n in range(2, 18):
        for op in ("sum", "avg", "max"):
            print("%s n=%d %s %s" % (sched, n, dtype, op), flush=True)
            count = n * 64 * u * 3 + u * 5 + 3
            xs = inputs(40, n, count, dtype, op)
            got = run_allreduce(xs, dtype, op, sched)
            want = oracle.ring_allreduce(xs, dtype, op)
            for r in (0, n - 1):
                assert_bits_equal(got[r], want[r], "%s ar n=%d %s %s rank %d" % (sched, n, dtype, op, r))
            R = 64 * u * 2 + u
            ys = inputs(41, n, n * R, dtype, op)
            got = run_rs(ys, dtype, op, sched)
            want = oracle.ring_reduce_scatter(ys, dtype, op)
            for r in range(n):
                assert_bits_equal(got[r], want[r], "%s rs n=%d %s %s rank %d" % (sched, n, dtype, op, r))
        # pieces of several two-run tiles plus a ragged tail; then slices off the vector grid (the phased
        # kernels, two 1 KB runs per lane up to 8 ranks) with several tiles per slice
        pieces = inputs(42, n, 64 * u * 5 + u, dtype, "sum")
        got = run_ag(pieces, dtype, sched)
        want = oracle.ring_all_gather(pieces, dtype)
        for r in (0, n - 1):
            assert_bits_equal(got[r], want[r], "%s ag n=%d %s rank %d" % (sched, n, dtype, r))
        Rp = 64 * u * 5 + 3
        ys = inputs(44, n, n * Rp, dtype, "sum")
        got = run_rs(ys, dtype, "sum", sched)
        want = oracle.ring_reduce_scatter(ys, dtype, "sum")
        for r in range(n):
            assert_bits_equal(got[r], want[r], "%s phased rs n=%d %s rank %d" % (sched, n, dtype, r))
        pieces = inputs(45, n, Rp, dtype, "sum")
        got = run_ag(pieces, dtype, sched)
        want = oracle.ring_all_gather(pieces, dtype)
        for r in (0, n - 1):
            assert_bits_equal(got[r], want[r], "%s phased ag n=%d %s rank %d" % (sched, n, dtype, r))


@pytest.mark.parametrize("sched", ["tree", "dtree"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_trees_every_rank_count_up_to_17(dtype, sched):
    """Every n up to 16 has its own compile-time tree kernels (17 takes the
    any-n path), for the single and the double binary tree."""
    u = LANES[dtype]
    for n in range(2, 18):
        for op in ("sum", "avg", "min"):
            print("%s n=%d %s %s" % (sched, n, dtype, op), flush=True)
            count = n * 64 * u * 5 + u * 7 + 3
            xs = inputs(43, n, count, dtype, op)
            got = run_allreduce(xs, dtype, op, sched)
            want = reference(sched, xs, dtype, op)
            for r in (0, n // 2, n - 1):
                assert_bits_equal(got[r], want[r], "%s n=%d %s %s rank %d" % (sched, n, dtype, op, r))


@pytest.mark.parametrize("teams", ["1", "0"])
def test_staged_trees_match_oracle(teams, monkeypatch):
    """The LDS-staged tree kernels (the streaming walk switched off), with
    concurrent up/down teams (teams=1) and level by level (teams=0), each
    forced: every dtype, ops whose order
    matters, rank counts up to 128 (n <= 16 through AR_TREE_STAGED), counts
    spanning many windows per workgroup with a ragged end, in and out of place,
    against the tree and double-tree oracles bit for bit."""
    monkeypatch.setenv("AR_TREE_STAGED", "1")
    monkeypatch.setenv("AR_TREE_STREAM", "0")
    monkeypatch.setenv("AR_TREE_TEAMS", teams)
    for n in (2, 3, 8, 16, 17, 33, 72, 128):
        for dtype in DTYPES:
            u = LANES[dtype]
            for op in (("sum", "avg", "max") if n in (17, 72) else ("avg",)):
                count = n * u * 600 + u * 5 + 3
                xs = inputs(61, n, count, dtype, op)
                for sched in ("tree", "dtree"):
                    for inplace in ((False, True) if n == 72 else (False,)):
                        print("staged %s teams=%s n=%d %s %s inplace=%d" % (sched, teams, n, dtype, op, inplace),
                              flush=True)
                        got = run_allreduce(xs, dtype, op, sched, inplace=inplace)
                        want = reference(sched, xs, dtype, op)
                        for r in (0, n // 2, n - 1):
                            assert_bits_equal(got[r], want[r], "staged %s teams=%s n=%d %s %s rank %d"
                                              % (sched, teams, n, dtype, op, r))


@pytest.mark.parametrize("dtype", DTYPES)
def test_streamed_trees_match_oracle(dtype, monkeypatch):
    """The streaming in-order walk of the trees, at rank counts whose walks
    differ: shallow and deep stacks, the mirror-image second tree (even n) and
    the shifted one walked from rank 1 (odd n; with reordered levels at 7, 19
    and 63 ranks), both
    tile shapes (below and from 64 ranks), n <= 16 through AR_TREE_STAGED, and
    127 ranks, whose shifted tree needs more stack than the walk holds and
    keeps the staged kernels.  Counts spanning several tiles with a ragged end,
    in and out of place, against the tree and double-tree oracles bit for bit."""
    monkeypatch.setenv("AR_TREE_STAGED", "1")
    monkeypatch.setenv("AR_TREE_STREAM", "1")                  # at every size (by default from 1 MB per rank)
    u = LANES[dtype]
    for n in (2, 3, 5, 7, 16, 17, 19, 24, 33, 63, 64, 65, 72, 100, 127, 128):
        tile = 64 * (8 if n >= 64 else 2)                      # vectors per tile
        count = (tile * 3 + 5) * u + 3
        for op in (OPS if n in (17, 65) else ("sum", "avg")):
            xs = inputs(70 + n, n, count, dtype, op)
            for sched in ("tree", "dtree"):
                want = reference(sched, xs, dtype, op)
                for inplace in ((False, True) if n in (33, 72) else (False,)):
                    print("streamed %s n=%d %s %s count=%d inplace=%d" % (sched, n, dtype, op, count, inplace),
                          flush=True)
                    got = run_allreduce(xs, dtype, op, sched, inplace=inplace)
                    for r in (0, n // 2, n - 1):
                        assert_bits_equal(got[r], want[r], "streamed %s n=%d %s %s rank %d inplace=%d"
                                          % (sched, n, dtype, op, r, inplace))


@pytest.mark.parametrize("n", [33, 100])
def test_streamed_trees_at_their_default_sizes(n, monkeypatch):
    """The walk as callers get it (no override): 2.5 MB per rank, so each half
    of the double tree is over the 1 MB-per-rank launch threshold; 33 ranks
    (2 KB runs with the residency reservation, the shifted second tree walked
    from rank 1) and 100 ranks (8 KB runs); fp32 avg and bf16 sum, against the
    tree and double-tree oracles bit for bit on every rank."""
    monkeypatch.delenv("AR_TREE_STREAM", raising=False)
    monkeypatch.delenv("AR_TREE_STAGED", raising=False)
    for dtype, op in (("f32", "avg"), ("bf16", "sum")):
        count = (5 << 19) // (4 if dtype == "f32" else 2) + LANES[dtype] * 3 + 1
        xs = inputs(90 + n, n, count, dtype, op)
        for sched in ("tree", "dtree"):
            print("default-size streamed %s n=%d %s %s count=%d" % (sched, n, dtype, op, count), flush=True)
            want = reference(sched, xs, dtype, op)
            got = run_allreduce(xs, dtype, op, sched)
            for r in range(n):
                assert_bits_equal(got[r], want[r], "default-size %s n=%d %s %s rank %d" % (sched, n, dtype, op, r))


def test_randomized_calls_match_oracle():
    """400 seeded random calls: collective, n (1-20 and 72), dtype, op,
    schedule, numerics options, element counts (log-uniform, ragged), in place
    or not, and each side's 16-byte phase (shared or mixed across ranks) --
    every combination of the library's paths (vector, shifted frame, phased,
    element-wise), each against the oracle bit for bit."""
    rng = np.random.default_rng(2024)
    for case in range(400):
        coll = rng.choice(["allreduce", "reduce_scatter", "all_gather"])
        n = int(rng.choice(list(range(1, 21)) + [72]))
        dtype = str(rng.choice(DTYPES))
        u = LANES[dtype]
        op = str(rng.choice(OPS)) if coll != "all_gather" else "sum"
        count = int(np.exp(rng.uniform(0, np.log(4096 if n > 20 else 40000))))
        mixed = rng.random() < 0.15
        ks = [int(rng.integers(u)) if mixed else 0 for _ in range(n)]
        k_in = int(rng.integers(u))
        k_out = int(rng.integers(u))
        if coll == "allreduce":
            scheds = ["fused", "ring", "tree", "dtree", "split", "auto"]
        else:
            scheds = ["fused", "ring", "auto"]
        sched = str(rng.choice(scheds))
        acc, avg = "storage", "prescale"
        if coll != "all_gather" and rng.random() < 0.2:
            acc, avg = NUMERICS[int(rng.integers(len(NUMERICS)))]
            if acc == "fp32" and dtype in ("bf16", "f16") and sched not in ("fused", "auto"):
                sched = "fused"
        inplace = coll == "allreduce" and not mixed and rng.random() < 0.3
        label = "case %d: %s n=%d %s %s count=%d sched=%s %s/%s in=%d out=%d mixed=%s inplace=%s" % (
            case, coll, n, dtype, op, count, sched, acc, avg, k_in, k_out, mixed, inplace)
        print(label, flush=True)
        if coll == "allreduce":
            xs = inputs(1000 + case, n, count, dtype, op)
            d_in = [_at_phase(x, dtype, (k_in + ks[r]) % u) for r, x in enumerate(xs)]
            d_out = d_in if inplace else [_at_phase(np.zeros_like(x), dtype, (k_out + ks[r]) % u)
                                          for r, x in enumerate(xs)]
            ar.ar_allreduce_ex(d_in, d_out, count, dtype, op, sched=sched, acc=acc, avg=avg)
            sync()
            used = sched
            if sched == "auto":
                used = "fused" if (acc == "fp32" and dtype in ("bf16", "f16")) else \
                    ar.ar_plan("allreduce", count, dtype, op, n).chosen
            ref = _numerics_reference(used, xs, dtype, op, acc, avg)
            for r in range(n):
                assert_bits_equal(to_host(d_out[r], dtype), ref[r], label + " rank %d" % r)
        elif coll == "reduce_scatter":
            R = max(1, count // max(n, 1))
            xs = inputs(1000 + case, n, n * R, dtype, op)
            d_in = [_at_phase(x, dtype, (k_in + ks[r]) % u) for r, x in enumerate(xs)]
            d_out = [_at_phase(np.zeros(R, dtype=xs[0].dtype), dtype, (k_out + ks[r]) % u) for r in range(n)]
            ar.ar_reduce_scatter_ex(d_in, d_out, R, dtype, op, sched=sched, acc=acc, avg=avg)
            sync()
            ref = _numerics_reference("ring", xs, dtype, op, acc, avg, coll="reduce_scatter")
            for r in range(n):
                assert_bits_equal(to_host(d_out[r], dtype), ref[r], label + " rank %d" % r)
        else:
            R = max(1, count // max(n, 1))
            pieces = inputs(1000 + case, n, R, dtype, "sum")
            d_in = [_at_phase(x, dtype, (k_in + ks[r]) % u) for r, x in enumerate(pieces)]
            d_out = [_at_phase(np.zeros(n * R, dtype=pieces[0].dtype), dtype, (k_out + ks[r]) % u) for r in range(n)]
            ar.ar_all_gather(d_in, d_out, R, dtype, sched=sched)
            sync()
            want = oracle.ring_all_gather(pieces, dtype)
            for r in range(n):
                assert_bits_equal(to_host(d_out[r], dtype), want[r], label + " rank %d" % r)
