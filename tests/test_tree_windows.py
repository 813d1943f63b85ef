"""Host model of the LDS-staged trees' window grid (CPU only).

The staged tree kernels walk windows of W vectors, W a multiple of 8 (whole
128-byte lines), over a range [lo, hi) on a grid from lo rounded down to a
multiple of W (the first window partial); the double tree is two launches,
[0, split) with the first tree and [split2, Vfull) with the second.  This
model restates the window arithmetic of the launcher and the kernels and
checks that every vector of both halves is covered exactly once, by a launch
of the right tree, and that every window starts on the grid.
"""
from __future__ import annotations

import random

ITEMS = 256 * 4          # threads per team x items per thread


def tree_window(n):
    w = ITEMS // (8 * n) * 8
    return max(w, 8)


def range_windows(lo, hi, W):
    base = lo - lo % W
    windows = (hi - base + W - 1) // W if hi > base else 0
    return base, windows


def covered_range(lo, hi, W, seen, tag):
    if lo >= hi:
        return
    base, windows = range_windows(lo, hi, W)
    for win in range(windows):
        pos0 = base + win * W
        assert pos0 % W == 0
        for v in range(pos0, pos0 + W):
            if lo <= v < hi:
                assert v not in seen, (v, win)
                seen[v] = tag


def covered(Vfull, split, split2, W, dual):
    seen = {}
    if dual:
        covered_range(0, split, W, seen, False)
        covered_range(split2, Vfull, W, seen, True)
    else:
        covered_range(0, Vfull, W, seen, False)
    return seen


def test_window_width_is_whole_lines_and_fits():
    for n in range(2, 129):
        W = tree_window(n)
        assert W % 8 == 0 and W >= 8
        assert n * W <= ITEMS


def test_single_tree_windows_cover_every_vector_once():
    rnd = random.Random(5)
    for _ in range(300):
        W = 8 * rnd.randint(1, 64)
        Vfull = rnd.randint(0, 5000)
        seen = covered(Vfull, Vfull, Vfull, W, False)
        assert sorted(seen) == list(range(Vfull))


def test_double_tree_windows_cover_both_halves_once():
    rnd = random.Random(7)
    for _ in range(600):
        W = 8 * rnd.randint(1, 64)
        Vfull = rnd.randint(0, 5000)
        split = rnd.randint(0, Vfull)
        split2 = min(Vfull, split + rnd.randint(0, 1))        # the shifted frame leaves one vector out
        seen = covered(Vfull, split, split2, W, True)
        want = list(range(split)) + list(range(split2, Vfull))
        assert sorted(seen) == want
        assert all(not seen[v] for v in range(split)) and all(seen[v] for v in range(split2, Vfull))
