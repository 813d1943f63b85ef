"""A second, independent CPU implementation of what the all-reduce path
computes -- TEST INFRASTRUCTURE ONLY (imported by the CPU tests, never by the
product library).

It shares nothing with ``oracle/``: no code, no table, no conversion routine.
Where ``oracle/`` is C that simulates the ring as messages moving between
per-rank wire buffers, this module is plain Python over numpy scalars that
evaluates, element by element, the expression each schedule defines:

* the ring ("NCCL all-reduce" post, sections "What all-reduce promises" and
  "The ring, exactly as the kernel runs it"): every rank's buffer is cut into
  n chunks; the partial of chunk c starts at rank c+1 and collects the
  contributions of ranks c+2, ..., c, each one added to the incoming total;
  rank c, where the chunk completes, applies the integer-avg division; the
  finished chunk is then copied unchanged to every rank;
* the tree (same post, section "The double binary tree"): the bit-trick
  parent map, a node's own value combined with its children's partials in
  ascending rank order, the root's value copied to every rank; the double
  binary tree with the mirrored (even n) or shifted (odd n) second tree on the
  second half of the buffer;
* every rank combined at once in the aligned pairwise order over rank indices
  (same post, section "When the switch does the math", whose order is left
  open);
* reduce-scatter and all-gather ("FSDP collectives 101", sections "Why
  backward needs a different collective" and "All-gather: everyone shows
  their piece");
* the two numerics trades of "FSDP collectives 101" (fp32 partials for
  bf16 / fp16; the fp16 average's divisor split between a pre-scale and a
  post-scale).

The readings where the pages are silent are the same ones ``oracle/`` takes
(chunk cut in 16-byte units with the floor of the M2N paper's Eq. (2);
chains from rank c+1 to rank c; incoming partial as the left operand;
min/max ties keep the incoming value; float avg multiplies by fp32(1/n);
every value leaving a hop rounded to the storage type; integer avg truncates
toward zero; int32 wraps).  Arithmetic: fp32 with numpy float32 scalars (one
IEEE operation each, nothing fused); bf16 rounding written here as round to
nearest even on the float32 bit pattern; fp16 rounding through numpy's
float32 -> float16 conversion; int32 with Python integers wrapped to 32 bits.
fp32(1/n) is chosen here as the float32 nearest to the exact fraction 1/n.

Slow on purpose: use it on buffers of at most a few thousand elements.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

_ELEM = {"f32": 4, "bf16": 2, "f16": 2, "i32": 4}


# ---------------------------------------------------------------------------
# values: storage bits <-> working values
# ---------------------------------------------------------------------------

def _bf16_round(v: np.float32) -> np.float32:
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    bits = int(np.float32(v).view(np.uint32))
    if (bits & 0x7F800000) == 0x7F800000 and (bits & 0x7FFFFF):
        return np.uint32((bits | 0x400000) & 0xFFFF0000).view(np.float32)      # NaN stays a quiet NaN
    keep_lsb = (bits >> 16) & 1
    bits = (bits + 0x7FFF + keep_lsb) & 0xFFFFFFFF
    return np.uint32(bits & 0xFFFF0000).view(np.float32)


def _to_storage_value(dtype: str, v):
    """Round a working value to the storage type (float types stay float32
    numbers exactly representable in the storage type)."""
    if dtype == "f32":
        return np.float32(v)
    if dtype == "bf16":
        return _bf16_round(np.float32(v))
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return np.float32(np.float16(np.float32(v)))
    raise ValueError(dtype)


def _read(dtype: str, arr, i):
    """Element i of a rank buffer as a working value."""
    if dtype == "i32":
        return int(arr[i])
    if dtype == "bf16":
        return np.uint32(int(arr[i]) << 16).view(np.float32)
    return np.float32(arr[i])


def _encode(dtype: str, values):
    if dtype == "i32":
        return np.array([((v + 2 ** 31) % 2 ** 32) - 2 ** 31 for v in values], dtype=np.int32)
    if dtype == "f32":
        return np.array(values, dtype=np.float32)
    if dtype == "f16":
        return np.array(values, dtype=np.float32).astype(np.float16)
    bits = np.array(values, dtype=np.float32).view(np.uint32)
    return (bits >> 16).astype(np.uint16)


def _wrap(v: int) -> int:
    return ((v + 2 ** 31) % 2 ** 32) - 2 ** 31


def nearest_f32(q: Fraction) -> np.float32:
    """The float32 nearest to the positive rational q (ties to even)."""
    f = np.float32(float(q))
    best = f
    for cand in (np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(np.inf))):
        d_best, d_cand = abs(Fraction(float(best)) - q), abs(Fraction(float(cand)) - q)
        if d_cand < d_best or (d_cand == d_best and int(cand.view(np.uint32)) % 2 == 0):
            best = cand
    return np.float32(best)


class _Numerics:
    """The per-call arithmetic: the op, the avg pre-scale and where values are
    rounded to the storage type."""

    def __init__(self, dtype: str, op: str, n: int, acc32: bool = False, avg_split: bool = False):
        self.dtype, self.op, self.n = dtype, op, n
        self.acc32 = acc32 and dtype in ("bf16", "f16")
        self.avg_split = avg_split and op == "avg" and dtype != "i32"
        self.p = 1
        if self.avg_split:
            while self.p * self.p < n:                  # least power of two p with p*p >= n
                self.p *= 2
        if op == "avg" and dtype != "i32":
            self.scale = nearest_f32(Fraction(1, self.p if self.avg_split else n))

    def contribution(self, v):
        """A rank's value as it is read (float avg: times fp32(1/n), one fp32 multiply)."""
        if self.op == "avg" and self.dtype != "i32":
            with np.errstate(over="ignore", under="ignore"):
                return np.float32(v) * self.scale
        return v

    def partial(self, v):
        """A value leaving a hop."""
        if self.dtype == "i32" or self.acc32:
            return v
        return _to_storage_value(self.dtype, v)

    def combine(self, incoming, own):
        op = self.op
        if self.dtype == "i32":
            if op in ("sum", "avg"):
                return _wrap(incoming + own)
            if op == "prod":
                return _wrap(incoming * own)
            if op == "min":
                return own if own < incoming else incoming
            return own if own > incoming else incoming
        with np.errstate(over="ignore", invalid="ignore"):
            if op in ("sum", "avg"):
                return np.float32(incoming) + np.float32(own)
            if op == "prod":
                return np.float32(incoming) * np.float32(own)
        if op == "min":
            return own if own < incoming else incoming
        return own if own > incoming else incoming

    def complete(self, v):
        """Where a reduction completes: integer avg divides once (truncating
        toward zero); the split float avg divides by n/p in fp32; the value is
        rounded to the storage type."""
        if self.dtype == "i32":
            if self.op == "avg":
                q = abs(v) // self.n
                return -q if v < 0 else q
            return v
        if self.avg_split:
            v = np.float32(v) / np.float32(self.n / self.p)          # n/p is exact in fp32
        return _to_storage_value(self.dtype, v)


# ---------------------------------------------------------------------------
# the ring
# ---------------------------------------------------------------------------

def chunk_bounds(dtype: str, n: int, count: int) -> list[int]:
    """All-reduce chunk c = [u*floor(c*V/n), u*floor((c+1)*V/n)) clamped to
    count, u = 16/element size, V = ceil(count/u)."""
    u = 16 // _ELEM[dtype]
    V = (count + u - 1) // u
    return [min(count, u * ((c * V) // n)) for c in range(n + 1)]


def _ring_chunk_value(xs, dtype, nm: _Numerics, c: int, i: int):
    """Element i of chunk c: start at rank c+1, add ranks c+2, ..., c."""
    n = len(xs)
    acc = nm.partial(nm.contribution(_read(dtype, xs[(c + 1) % n], i)))
    for k in range(2, n + 1):
        own = nm.contribution(_read(dtype, xs[(c + k) % n], i))
        acc = nm.partial(nm.combine(acc, own))
    return nm.complete(acc)


def ring_allreduce(xs, dtype: str, op: str, acc32: bool = False, avg_split: bool = False):
    """Every rank's output (one array; the all-gather copies it unchanged)."""
    n, count = len(xs), len(xs[0])
    nm = _Numerics(dtype, op, n, acc32, avg_split)
    off = chunk_bounds(dtype, n, count)
    out = [None] * count
    for c in range(n):
        for i in range(off[c], off[c + 1]):
            out[i] = _ring_chunk_value(xs, dtype, nm, c, i)
    return _encode(dtype, out)


def ring_reduce_scatter(xs, dtype: str, op: str, acc32: bool = False, avg_split: bool = False):
    """Rank r keeps slice r (the equal split of its n*R input elements)."""
    n = len(xs)
    R = len(xs[0]) // n
    nm = _Numerics(dtype, op, n, acc32, avg_split)
    return [_encode(dtype, [_ring_chunk_value(xs, dtype, nm, r, r * R + i) for i in range(R)]) for r in range(n)]


def all_gather(xs):
    """Every rank receives x_0 || x_1 || ... || x_{n-1}, bit for bit."""
    return np.concatenate(list(xs))


# ---------------------------------------------------------------------------
# the trees
# ---------------------------------------------------------------------------

def tree_parent(n: int, v: int) -> int:
    """Bit-trick parent: clear v's lowest set bit b and set bit 2b; past the end
    of the range, only clear b.  Rank 0 is the root (-1)."""
    if v == 0:
        return -1
    b = v & (-v)
    p = (v & ~b) | (b << 1)
    return p if p < n else v & ~b


def second_tree_parent(n: int, v: int) -> int:
    """The double tree's other tree: the mirror image (rank v in rank n-1-v's
    place) for even n, the first tree moved up by one rank for odd n."""
    if n % 2 == 0:
        p = tree_parent(n, n - 1 - v)
        return -1 if p < 0 else n - 1 - p
    p = tree_parent(n, (v - 1) % n)
    return -1 if p < 0 else (p + 1) % n


def _children(n: int, parent) -> dict:
    kids = {v: [] for v in range(n)}
    for v in range(n):
        p = parent(n, v)
        if p >= 0:
            kids[p].append(v)
    return {v: sorted(k) for v, k in kids.items()}


def _tree_value(xs, dtype, nm: _Numerics, kids, root, i):
    """Up the tree: a node's own value, then each child's partial in ascending
    rank order; the root's value is every rank's result."""

    def up(v):
        acc = nm.partial(nm.contribution(_read(dtype, xs[v], i)))
        for ch in kids[v]:
            acc = nm.partial(nm.combine(acc, up(ch)))
        return acc

    return nm.complete(up(root))


def tree_allreduce(xs, dtype: str, op: str, acc32: bool = False, avg_split: bool = False):
    n, count = len(xs), len(xs[0])
    nm = _Numerics(dtype, op, n, acc32, avg_split)
    kids = _children(n, tree_parent)
    return _encode(dtype, [_tree_value(xs, dtype, nm, kids, 0, i) for i in range(count)])


def dtree_allreduce(xs, dtype: str, op: str, acc32: bool = False, avg_split: bool = False):
    """Elements [0, u*floor(V/2)) up the first tree, the rest up the second."""
    n, count = len(xs), len(xs[0])
    nm = _Numerics(dtype, op, n, acc32, avg_split)
    u = 16 // _ELEM[dtype]
    half = u * (((count + u - 1) // u) // 2)
    root2 = [v for v in range(n) if second_tree_parent(n, v) < 0][0]
    kids1, kids2 = _children(n, tree_parent), _children(n, second_tree_parent)
    out = [_tree_value(xs, dtype, nm, kids1, 0, i) if i < half
           else _tree_value(xs, dtype, nm, kids2, root2, i) for i in range(count)]
    return _encode(dtype, out)


# ---------------------------------------------------------------------------
# every rank at once, in the aligned pairwise order
# ---------------------------------------------------------------------------

def pairwise_reduce(xs, dtype: str, op: str, acc32: bool = False, avg_split: bool = False):
    n, count = len(xs), len(xs[0])
    nm = _Numerics(dtype, op, n, acc32, avg_split)

    def part(lo, ln, i):
        if ln == 1:
            return nm.partial(nm.contribution(_read(dtype, xs[lo], i)))
        h = 1 << ((ln - 1).bit_length() - 1)            # the largest power of two below ln
        return nm.partial(nm.combine(part(lo, h, i), part(lo + h, ln - h, i)))

    return _encode(dtype, [nm.complete(part(0, n, i)) for i in range(count)])
