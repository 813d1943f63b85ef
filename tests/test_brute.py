"""The oracle against a second, independent implementation (``tests/brute.py``),
bit for bit, on random data whose floating-point results depend on the order
of operations: every schedule's expression, every dtype and op (avg
included), rank counts 1-9, 16, 17 and 72, counts that the 16-byte chunk cut
leaves ragged, and both numerics variants.  CPU only.

The hand-derived cases in ``test_oracle.py`` fix the readings (hop order,
floor chunk cut, avg pre-scale); this file checks that the oracle's C carries
them out on general data exactly as a plain evaluation of the pages' steps
does, so a slip in either implementation shows as a mismatch.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import brute
import oracle
import workloads

DTYPES = ["f32", "bf16", "f16", "i32"]
OPS = ["sum", "prod", "min", "max", "avg"]
ELEM = {"f32": 4, "bf16": 2, "f16": 2, "i32": 4}


def rank_data(dtype, op, n, count, seed):
    """Order-sensitive test data: N(0,1) for sums and averages (1 % of entries
    x100), values near +-1 for products, wide integers for int32 (sums wrap)."""
    out = []
    for r in range(n):
        if dtype == "i32":
            lo, hi = ((-5, 5) if op == "prod" else (-(1 << 30), 1 << 30))
            out.append(workloads.ints(seed, 0, r, count, lo, hi, "i32"))
            continue
        if op == "prod":
            v = workloads.uniform(seed, 0, r, count, 0.7, 1.4, "f32")
            v = v * np.where(workloads.rng(seed, 1, r).random(count) < 0.5, -1, 1).astype(np.float32)
        else:
            v = workloads.normal(seed, 0, r, count, 1.0, "f32")
            v = v * np.where(workloads.rng(seed, 2, r).random(count) < 0.01, 100, 1).astype(np.float32)
        if dtype == "f32":
            out.append(v.astype(np.float32))
        elif dtype == "f16":
            out.append(v.astype(np.float16))
        else:
            out.append(brute._encode("bf16", [brute._bf16_round(np.float32(x)) for x in v]))
    return out


def counts(dtype, n):
    u = 16 // ELEM[dtype]
    c = {0, 1, 7, 37, u * n + 3, u * n - 1}
    if n <= 9:
        c.add(2 * u * n + u - 1)
    return sorted(x for x in c if x >= 0)


def same(a, b, what):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    if a.tobytes() == b.tobytes():
        return
    if a.shape == b.shape and a.itemsize == b.itemsize:
        bad = np.flatnonzero((a.view(np.uint8).reshape(a.size, -1) != b.view(np.uint8).reshape(b.size, -1)).any(1))
        raise AssertionError("%s: oracle and brute differ in %d elements, first %s" % (what, bad.size, bad[:5].tolist()))
    raise AssertionError("%s: oracle and brute differ in shape or type" % (what,))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
def test_every_schedule_matches_the_brute_evaluation(dtype, op):
    for n in (1, 2, 3, 4, 5, 6, 7, 8, 9, 16, 17):
        for count in counts(dtype, n):
            xs = rank_data(dtype, op, n, count, 100 + n)
            tag = (dtype, op, n, count)
            want = brute.ring_allreduce(xs, dtype, op)
            for r, y in enumerate(oracle.ring_allreduce(xs, dtype, op)):
                same(y, want, ("ring",) + tag + (r,))
            want = brute.tree_allreduce(xs, dtype, op)
            for y in oracle.tree_allreduce(xs, dtype, op):
                same(y, want, ("tree",) + tag)
            want = brute.dtree_allreduce(xs, dtype, op)
            for y in oracle.dtree_allreduce(xs, dtype, op):
                same(y, want, ("dtree",) + tag)
            same(oracle.pairwise_reduce(xs, dtype, op), brute.pairwise_reduce(xs, dtype, op), ("pairwise",) + tag)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
def test_reduce_scatter_and_all_gather_match_the_brute_evaluation(dtype, op):
    for n in (1, 2, 3, 5, 8, 9, 17):
        for R in (0, 1, 3, 5, 9):
            xs = rank_data(dtype, op, n, n * R, 200 + n)
            got = oracle.ring_reduce_scatter(xs, dtype, op)
            want = brute.ring_reduce_scatter(xs, dtype, op)
            for r in range(n):
                same(got[r], want[r], ("rs", dtype, op, n, R, r))
            cat = brute.all_gather(want)
            for y in oracle.ring_all_gather(got, dtype):
                same(y, cat, ("ag", dtype, n, R))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i32"])
def test_72_ranks_match_the_brute_evaluation(dtype):
    """The bucketed workload's rank count: 72 chunks of uneven length (the
    count is not a multiple of 72 vectors), avg and sum."""
    u = 16 // ELEM[dtype]
    for op in ("avg", "sum", "max"):
        count = u * 72 + 2 * u + 3
        xs = rank_data(dtype, op, 72, count, 72)
        assert len(set(np.diff(brute.chunk_bounds(dtype, 72, count)).tolist())) > 1
        want = brute.ring_allreduce(xs, dtype, op)
        for r, y in enumerate(oracle.ring_allreduce(xs, dtype, op)):
            same(y, want, ("ring72", dtype, op, r))
        same(oracle.pairwise_reduce(xs, dtype, op), brute.pairwise_reduce(xs, dtype, op), ("pairwise72", dtype, op))
        same(oracle.tree_allreduce(xs, dtype, op)[0], brute.tree_allreduce(xs, dtype, op), ("tree72", dtype, op))
    xs = rank_data(dtype, "avg", 72, 72 * 2, 73)
    got = oracle.ring_reduce_scatter(xs, dtype, "avg")
    want = brute.ring_reduce_scatter(xs, dtype, "avg")
    for r in range(72):
        same(got[r], want[r], ("rs72", dtype, r))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_numerics_variants_match_the_brute_evaluation(dtype):
    for n in (2, 3, 8, 9, 17):
        for op in ("sum", "avg", "prod"):
            for acc32, split in ((True, False), (False, True), (True, True)):
                if split and op != "avg":
                    continue
                count = (16 // ELEM[dtype]) * n + 5
                xs = rank_data(dtype, op, n, count, 300 + n)
                tag = (dtype, n, op, acc32, split)
                want = brute.ring_allreduce(xs, dtype, op, acc32, split)
                same(oracle.ring_allreduce(xs, dtype, op, acc32=acc32, avg_split=split)[0], want, ("ring",) + tag)
                same(oracle.tree_allreduce(xs, dtype, op, acc32=acc32, avg_split=split)[0],
                     brute.tree_allreduce(xs, dtype, op, acc32, split), ("tree",) + tag)
                same(oracle.pairwise_reduce(xs, dtype, op, acc32=acc32, avg_split=split),
                     brute.pairwise_reduce(xs, dtype, op, acc32, split), ("pairwise",) + tag)


def test_extreme_values_match_the_brute_evaluation():
    """Subnormals and sums that overflow to infinity, every float type."""
    for dtype in ("f32", "bf16", "f16"):
        for n in (2, 3, 8, 17):
            count = 16 // ELEM[dtype] * n + 9
            xs = [workloads.extremes(400, 0, r, count, dtype) for r in range(n)]
            for op in ("sum", "avg", "prod", "min", "max"):
                same(oracle.ring_allreduce(xs, dtype, op)[0], brute.ring_allreduce(xs, dtype, op), (dtype, n, op))


def test_brute_chunk_bounds_and_scale_agree_with_the_hand_cases():
    """The brute evaluation's own readings against the hand-evaluated values
    (the floor cut of the chunk bounds; fp32(1/n) as the nearest float)."""
    assert brute.chunk_bounds("f32", 3, 20) == [0, 4, 12, 20]
    assert brute.chunk_bounds("bf16", 5, 30) == [0, 0, 8, 16, 24, 30]
    assert brute.chunk_bounds("i32", 8, 100) == [0, 12, 24, 36, 48, 60, 72, 84, 100]
    assert int(brute.nearest_f32(Fraction(1, 3)).view(np.uint32)) == 0x3EAAAAAB
    assert int(brute.nearest_f32(Fraction(1, 72)).view(np.uint32)) == 0x3C638E39
    for n in range(1, 129):
        # the nearest float to 1/n is what a double 1/n rounded to float gives (no double rounding at these n)
        assert brute.nearest_f32(Fraction(1, n)) == np.float32(1.0 / n), n
