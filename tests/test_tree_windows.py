"""Host model of the LDS-staged trees' window grid (CPU only).

The staged tree and double-tree kernels walk windows of W vectors, W a
multiple of 8 (whole 128-byte lines), on a grid from vector 0; the double
tree's second half [split2, Vfull) starts at split2 rounded down to the grid,
its first window partial.  This model restates the window arithmetic of the
kernels and the host's window count and checks that every vector of
[0, split) and [split2, Vfull) is covered exactly once, by a window of the
right tree, and that every window starts on the grid.
"""
from __future__ import annotations

import random

ITEMS = 256 * 4          # threads per team x items per thread


def tree_window(n):
    w = ITEMS // (8 * n) * 8
    return max(w, 8)


def dtree_windows(Vfull, split, split2, W):
    base = split2 - split2 % W
    return (split + W - 1) // W + ((Vfull - base + W - 1) // W if Vfull > base else 0)


def window_at(win, first, Vfull, split, split2, W, dual):
    second = dual and win >= first
    pos0 = split2 - split2 % W + (win - first) * W if second else win * W
    lo = split2 if second else 0
    hi = split if dual and not second else Vfull
    return pos0, lo, hi, second


def covered(Vfull, split, split2, W, dual):
    windows = dtree_windows(Vfull, split, split2, W) if dual else (Vfull + W - 1) // W
    first = (split + W - 1) // W if dual else windows
    seen = {}
    for win in range(windows):
        pos0, lo, hi, second = window_at(win, first, Vfull, split, split2, W, dual)
        assert pos0 % W == 0
        for v in range(pos0, pos0 + W):
            if lo <= v < hi:
                assert v not in seen, (v, win)
                seen[v] = second
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
