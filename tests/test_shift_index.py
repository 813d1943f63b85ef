"""Host model of the shifted-frame all-reduce index arithmetic.

When every send and receive buffer sits at one 16-byte phase (not zero), the
all-reduce's vector kernels run on the pointers advanced by ``head`` elements
to the first 16-byte boundary, with the chunks and the double tree's split
still those of element index 0 (api.cpp, fused.hip, ring.hip, tree_reg.hip).
The fused and ring kernels end each chunk one frame vector early; the double
tree sends frame vectors [0, S - 1) up the first tree and [S, Vfull) up the
second; the element-wise kernels take the rest (elem.hip: in ring order each
chunk's first elements, the frame vector across its end and the tail; in
tree and split order the head, the vector across the split and the tail).

This file restates those index maps and checks, for every schedule, rank
count, element size, phase and many counts, that every element of [0, count)
is written exactly once, and that every frame vector a ring-order kernel
combines lies wholly inside one chunk (its hop order is the chunk's).  It
models the arithmetic only; the GPU parity tests check the values.
"""
import random

import pytest


def chunk_start(c, V, n):
    return (c * V) // n


def coverage(n, count, e, head, sched, early=1):
    """Write count per element of one call; ``early`` is how many frame vectors the ring-order kernels stop
    short of each chunk's end (1 in the library; 0 plants a mistake)."""
    u = 16 // e
    V = (count + u - 1) // u
    Vf = (count - head) // u
    S = V // 2
    split = min(S - 1, Vf) if S >= 1 else 0
    split2 = min(S, Vf)
    cov = [0] * count

    def mark(a, b):
        for i in range(a, b):
            assert 0 <= i < count
            cov[i] += 1

    if sched in ("fused", "ring"):
        for c in range(n):
            b0, b1 = chunk_start(c, V, n), chunk_start(c + 1, V, n)
            vend = min(b1 - early, Vf)
            for j in range(b0, vend):
                mark(head + u * j, head + u * j + u)
                for i in (head + u * j, head + u * j + u - 1):      # the vector lies inside chunk c
                    assert u * b0 <= i < u * b1, (n, count, e, head, c, j)
            lo, hi = u * b0, min(u * b1, count)
            fe = min(b1 - 1, Vf)
            s0 = head + u * b0
            s1 = head + u * fe if fe > b0 else s0
            a1, a2 = min(s0, hi), max(s1, lo)
            if a1 > lo:
                mark(lo, a1)
            if hi > a2:
                mark(a2, hi)
    else:
        if sched == "dtree":
            for j in range(0, split):
                mark(head + u * j, head + u * j + u)
                assert head + u * j + u <= u * S
            for j in range(split2, Vf):
                mark(head + u * j, head + u * j + u)
                assert head + u * j >= u * S
        else:
            for j in range(Vf):
                mark(head + u * j, head + u * j + u)
        end = head + u * Vf
        ranges = [(0, head), (head + u * split, head + u * split2 if sched == "dtree" else head + u * split),
                  (end, count)]
        for a, b in ranges:
            if b > a:
                mark(a, b)
    return cov


@pytest.mark.parametrize("sched", ["fused", "ring", "tree", "dtree", "split"])
def test_shifted_frame_partitions_every_count(sched):
    rng = random.Random(5)
    for n in (2, 3, 5, 8, 16, 17, 72):
        for e in (2, 4):
            u = 16 // e
            for head in range(1, u):
                counts = list(range(head + 1, head + 2 * u * n + 5, 3)) + [rng.randrange(head + 1, 3000)
                                                                          for _ in range(6)]
                for count in counts:
                    cov = coverage(n, count, e, head, sched)
                    assert all(x == 1 for x in cov), (sched, n, count, e, head)


def test_model_notices_a_chunk_that_ends_late():
    """Without the early end, some frame vector straddles two chunks (or an element is written twice)."""
    caught = 0
    for n in (3, 8):
        for count in range(10, 300, 7):
            try:
                cov = coverage(n, count, 4, 1, "fused", early=0)
                caught += int(not all(x == 1 for x in cov))
            except AssertionError:
                caught += 1
    assert caught > 0
