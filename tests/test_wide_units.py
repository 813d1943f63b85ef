"""Host model of the wide fused all-reduce's grid (n > 16; CPU only).

Chunk c is frame vectors [lo, hi): the floor cut lo = c*q + floor(c*rem/n),
hi = the next start less ``shift`` (the shifted frame leaves the vector
across each boundary to the element-wise kernel), clamped to Vfull.  Each
chunk is cut on a tile grid of T vectors aligned to ``ref``; a tile across
the boundary of chunks c and c+1 that is whole, inside [0, Vfull) and holds
no third chunk is one unit walking both chunks' hop orders, counted with
chunk c.  The grid is one workgroup per unit in address order, first[c]
units before chunk c, and a workgroup finds its chunk by binary search.

This model restates that arithmetic (the launcher's unit count and the
kernel's unit -> tile map) and checks, over many small geometries, that
every vector of every chunk is produced exactly once, by its own chunk's
hop order, and never the shifted frame's boundary vectors; that shared
tiles hold exactly two chunks; and that the grid has no empty unit.
"""
from __future__ import annotations

import itertools


def chunk_start(c, V, n):
    q, rem = divmod(V, n)
    return c * q + (c * rem) // n


def chunk(c, V, n, Vfull, shift):
    lo = chunk_start(c, V, n)
    hi = min(chunk_start(c + 1, V, n) - shift, Vfull)
    return lo, hi


def tiles(ref, lo, hi, T):
    return (ref + hi + T - 1) // T - (ref + lo) // T if hi > lo else 0


def shared(c, V, n, Vfull, shift, ref, T):
    """First vector of the shared tile across chunks c and c+1, or None."""
    if c + 1 >= n:
        return None
    b = chunk_start(c + 1, V, n)
    m = (ref + b) % T
    if m <= shift:
        return None
    ts = b - m
    lo, _ = chunk(c, V, n, Vfull, shift)
    _, hi1 = chunk(c + 1, V, n, Vfull, shift)
    return ts if ts >= lo and ts + T <= hi1 else None


def first_units(V, n, Vfull, shift, ref, T):
    first, total = [], 0
    for c in range(n):
        first.append(total)
        lo, hi = chunk(c, V, n, Vfull, shift)
        total += tiles(ref, lo, hi, T) - (1 if c > 0 and shared(c - 1, V, n, Vfull, shift, ref, T) is not None else 0)
    return first + [total], total


def unit_vectors(p, first, V, n, Vfull, shift, ref, T):
    """(vector, chunk) pairs one workgroup produces."""
    lo_c, hi_c = 0, n                                  # binary search: first[c] <= p < first[c+1]
    while hi_c - lo_c > 1:
        mid = (lo_c + hi_c) // 2
        if first[mid] <= p:
            lo_c = mid
        else:
            hi_c = mid
    c = lo_c
    cl, ch = chunk(c, V, n, Vfull, shift)
    j = p - first[c] + (1 if c > 0 and shared(c - 1, V, n, Vfull, shift, ref, T) is not None else 0)
    ts = shared(c, V, n, Vfull, shift, ref, T)
    if ts is not None and j == tiles(ref, cl, ch, T) - 1:
        b = chunk_start(c + 1, V, n)
        out = []
        for v in range(ts, ts + T):
            if shift and v == b - 1:
                continue                               # the element-wise kernel's vector
            out.append((v, c if v < b else c + 1))
        return out
    start = cl - (ref + cl) % T + j * T
    return [(v, c) for v in range(max(start, cl), min(start + T, ch))]


def check(V, n, Vfull, shift, ref, T):
    first, total = first_units(V, n, Vfull, shift, ref, T)
    seen = {}
    for p in range(total):
        got = unit_vectors(p, first, V, n, Vfull, shift, ref, T)
        assert got, "empty unit %d (V=%d n=%d shift=%d ref=%d)" % (p, V, n, shift, ref)
        for v, c in got:
            assert v not in seen, "vector %d twice" % v
            seen[v] = c
    want = {}
    for c in range(n):
        lo, hi = chunk(c, V, n, Vfull, shift)
        for v in range(lo, hi):
            want[v] = c
    assert seen == want, "V=%d n=%d shift=%d ref=%d T=%d" % (V, n, shift, ref, T)


def test_every_vector_once_in_its_own_chunk_order():
    T = 16
    for n, V, shift, ref in itertools.product((17, 18, 24, 33), (0, 1, 17, 40, 255, 256, 257, 700, 1601),
                                              (0, 1), (0, 1, 5, 15)):
        Vfull = V - (1 if shift and V else 0)          # the shifted frame ends a vector early
        check(V, n, max(Vfull, 0), shift, ref, T)


def test_shared_tiles_hold_exactly_two_chunks():
    T = 16
    for n, V, shift, ref in itertools.product((17, 20, 72), (300, 1000, 5000), (0, 1), range(0, 16, 3)):
        Vfull = V - shift
        for c in range(n - 1):
            ts = shared(c, V, n, Vfull, shift, ref, T)
            if ts is None:
                continue
            owners = {cc for cc in range(n) for v in range(ts, ts + T)
                      if chunk(cc, V, n, Vfull, shift)[0] <= v < chunk(cc, V, n, Vfull, shift)[1]}
            assert owners == {c, c + 1}, (n, V, shift, ref, c, owners)


def test_bucket_shape_uses_one_unit_per_tile():
    """A 25 MB fp32 bucket at 72 ranks (6,253,952 elements, 16 KB tiles): the
    shared tiles make the unit count the number of grid tiles the buffer
    touches, not that plus one per chunk boundary."""
    T, n = 1024, 72
    V = 6253952 // 4
    for ref in (0, 1, 777):
        first, total = first_units(V, n, V, 0, ref, T)
        grid_tiles = (ref + V + T - 1) // T - ref // T
        boundaries_on_grid = sum(1 for c in range(1, n) if (ref + chunk_start(c, V, n)) % T == 0)
        assert total == grid_tiles, (ref, total, grid_tiles, boundaries_on_grid)
