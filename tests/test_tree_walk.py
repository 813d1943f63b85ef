"""Host model of the streaming tree walk (CPU only).

The tree schedules combine, at every rank, its own value and then its
children's partials in ascending rank order, the root's partial being the
result.  The streaming kernel visits the ranks once each, from rank
``first`` upward and around, and keeps partials on a stack.  At each step a
program word says: combine the partial on top (the child visited before), keep
the partial pending (a child still to come), or finish the subtree and, for
``levels`` ancestors, combine it into the ancestor's pending partial (popping
also, where the ancestor's lower-rank child is the one visited last, the other
child's partial that the ancestor left under its own).

This model restates how the program is derived (run on node ids, every pop
checked) and how the kernel evaluates it, and checks on symbolic values, for
both trees of the double-tree schedule at every rank count up to 128, that the
walk gives exactly the tree's combine order within seven stack slots.  The
trees come from the oracle's definition.  The one tree the walk cannot hold is
the shifted second tree at 127 ranks (eight slots), which keeps the staged
kernels.
"""
from __future__ import annotations

import oracle

SLOTS = 7


def children(n, which):
    par = [oracle.dtree_parent(n, which, v) for v in range(n)]
    ch = [sorted(c for c in range(n) if par[c] == p) for p in range(n)]
    return par, ch


def program(n, which, first):
    """Program words (below, pending, [swap per level]) or None, and the stack depth."""
    par, ch = children(n, which)
    pos = {(first + v) % n: v for v in range(n)}
    stack, prog, depth = [], [], 0

    def pop(want):
        return bool(stack) and stack.pop() == want

    for v in range(n):
        r = (first + v) % n
        before = [c for c in ch[r] if pos[c] < v]
        after = [c for c in ch[r] if pos[c] > v]
        if len(before) > 1 or len(after) > 1:
            return None, depth
        keep = bool(before and after and after[0] == ch[r][0])
        if before and not keep and not pop(("done", before[0])):
            return None, depth
        levels = []
        if after:
            if keep and not (stack and stack[-1] == ("done", before[0])):
                return None, depth
            stack.append(("pending", r))
        else:
            x = r
            while par[x] >= 0 and pos[par[x]] < pos[x]:
                p = par[x]
                if not pop(("pending", p)):
                    return None, depth
                swap = ch[p][0] == x and len(ch[p]) == 2
                if swap and not pop(("done", ch[p][1])):
                    return None, depth
                levels.append(swap)
                x = p
            stack.append(("done", x))
        depth = max(depth, len(stack))
        prog.append((r, bool(before) and not keep, bool(after), levels))
    if stack != [("done", par.index(-1))]:
        return None, depth
    return prog, depth


def walk(prog, own):
    """The kernel's evaluation (``(a, b)`` is a combined with b, a the
    accumulator); None when the program leaves the stack in any other state
    than one partial."""
    stack = []
    for r, below, pending, levels in prog:
        acc = own[r]
        if below:
            if not stack:
                return None
            acc = (acc, stack.pop())
        if not pending:
            for swap in levels:
                if len(stack) < 1 + swap:
                    return None
                acc = (stack.pop(), acc)
                if swap:
                    acc = (acc, stack.pop())
        stack.append(acc)
    return stack[0] if len(stack) == 1 else None


def tree_order(n, which, own):
    par, ch = children(n, which)

    def part(v):
        acc = own[v]
        for c in ch[v]:
            acc = (acc, part(c))
        return acc
    return part(par.index(-1))


def test_walk_reproduces_every_tree_up_to_128_ranks():
    held_back = []
    for n in range(1, 129):
        own = ["x%d" % v for v in range(n)]
        for which in (0, 1):
            firsts = (1,) if which == 1 and n % 2 == 1 else (0,)
            for first in firsts:
                prog, depth = program(n, which, first)
                if prog is None or depth > SLOTS:
                    held_back.append((n, which))
                    continue
                assert walk(prog, own) == tree_order(n, which, own), (n, which)
    assert held_back == [(127, 1)]


def test_shifted_tree_is_not_walkable_from_rank_0():
    """Odd n: the second tree wraps rank n-1's place onto rank 0, so the walk
    from rank 0 is refused (the kernel starts that tree at rank 1)."""
    for n in (3, 5, 17, 33, 65):
        assert program(n, 1, 0)[0] is None


def test_walk_catches_a_misordered_program():
    """A program with one level's reorder flag dropped gives a different
    combine order: the symbolic check is sensitive to it.  (The shifted tree
    reorders a level at 7, 11, 13, 15, 19, ... ranks, not at 17 or 33.)"""
    n = 19
    prog, _ = program(n, 1, 1)
    own = ["x%d" % v for v in range(n)]
    flipped = False
    for i, (r, below, pending, levels) in enumerate(prog):
        if any(levels):
            prog[i] = (r, below, pending, [False] * len(levels))
            flipped = True
            break
    assert flipped
    assert walk(prog, own) != tree_order(n, 1, own)
    assert walk(program(n, 1, 1)[0], own) == tree_order(n, 1, own)
