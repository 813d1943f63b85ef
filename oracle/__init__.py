"""CPU oracle for the n-rank all-reduce path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``reduce_scatter_amd``) never imports it, and this package imports nothing
from the product: the two share no code.

The arithmetic lives in ``ar_oracle.c`` (plain C, built with gcc and
``-ffp-contract=off``); this module only marshals numpy arrays to it.  The
functions follow:

* "NCCL all-reduce" post (rakshithvasudev.github.io), sections "What
  all-reduce promises" and "The ring, exactly as the kernel runs it":
  :func:`ring_allreduce`, :func:`ring_reduce_scatter`, :func:`ring_all_gather`;
  section "The double binary tree": :func:`tree_parent`, :func:`tree_allreduce`,
  and the two complementary trees: :func:`dtree_parent`, :func:`dtree_allreduce`;
  the plain element-wise definition (exact for int32 and min/max):
  :func:`direct_reduce`; section "When the switch does the math" (every rank
  combined at once, in an order the post leaves open; read as the aligned
  pairwise tree over rank indices): :func:`pairwise_reduce`.
* "FSDP collectives 101", the notes that bf16 reductions accumulate in bf16
  (hence reducing in fp32) and that fp16 averages split the divisor across pre-
  and post-scaling: the ``acc32`` and ``avg_split`` options (:func:`split_p`).
* "FSDP collectives 101" (rakshithvasudev.github.io), sections "All-gather:
  everyone shows their piece" and "Why backward needs a different collective":
  the semantics of reduce-scatter (rank r keeps slice r) and all-gather.

The M-to-N layout reshard of the "NCCL M2N" paper (arxiv.org/html/2610.07516)
has its own oracle in :mod:`oracle.reshard` (plain numpy: layouts, Eq. (1)
and (2), the reshard's definition, the §V-A schedule and §V-B leaders).

Array conventions: ``f32`` arrays are ``np.float32``, ``f16`` arrays are
``np.float16``, ``i32`` arrays are ``np.int32`` and ``bf16`` arrays are
``np.uint16`` holding the bfloat16 bit patterns.

Parity status: every function here is pinned by ``tests/test_oracle.py``
(worked examples from the pages, exact brute force, closed forms and
hand-derived rounding cases, hand-evaluated chunk bounds at counts n does not
divide and hand-evaluated avg pre-scales at n = 3 and 72), agrees bit for bit
with the independent evaluation in ``tests/brute.py`` on order-sensitive
random data, and ``tests/test_oracle_mutants.py`` shows planted mistakes in
``ar_oracle.c`` failing those pins.  The exact floating-point hop order inside
a chunk is a reading (chunk c starts at rank c+1 and ends at rank c); the
pages' step diagrams were lost, so that order is pinned by hand-derived cases
built from the reading, not by a printed example.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ar_oracle.c")
_LIB = os.path.join(_HERE, "libar_oracle.so")

DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2, "i32": 3}
NP_DTYPE = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16, "i32": np.int32}
OP_CODE = {"sum": 0, "prod": 1, "min": 2, "max": 3, "avg": 4}

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile ``ar_oracle.c`` into ``libar_oracle.so`` with gcc."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
        return _lib


def _bind(lib):
    """Declare the C functions' argument and result types on a loaded oracle library."""
    vpp = ctypes.POINTER(ctypes.c_void_p)
    llp = ctypes.POINTER(ctypes.c_longlong)
    for name in ("orc_ring_allreduce_ex", "orc_ring_reduce_scatter_ex"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_size_t, vpp, vpp, llp, llp,
                      ctypes.c_int, ctypes.c_int]
        f.restype = ctypes.c_int
    for name in ("orc_tree_allreduce_ex", "orc_dtree_allreduce_ex"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_size_t, vpp, vpp, ctypes.c_int, ctypes.c_int]
        f.restype = ctypes.c_int
    lib.orc_pairwise_reduce_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_size_t, vpp,
                                           ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
    lib.orc_pairwise_reduce_ex.restype = ctypes.c_int
    lib.orc_split_p.argtypes = [ctypes.c_int]
    lib.orc_split_p.restype = ctypes.c_int
    lib.orc_ring_all_gather.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_size_t, vpp, vpp, llp, llp]
    lib.orc_ring_all_gather.restype = ctypes.c_int
    lib.orc_tree_allreduce.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_size_t, vpp, vpp]
    lib.orc_tree_allreduce.restype = ctypes.c_int
    lib.orc_direct_reduce.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_size_t, vpp,
                                      ctypes.c_void_p]
    lib.orc_direct_reduce.restype = ctypes.c_int
    lib.orc_pairwise_reduce.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_size_t, vpp,
                                        ctypes.c_void_p]
    lib.orc_pairwise_reduce.restype = ctypes.c_int
    lib.orc_dtree_allreduce.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_size_t, vpp, vpp]
    lib.orc_dtree_allreduce.restype = ctypes.c_int
    lib.orc_dtree_parent.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.orc_dtree_parent.restype = ctypes.c_int
    lib.orc_tree_parent.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.orc_tree_parent.restype = ctypes.c_int
    lib.orc_allreduce_chunks.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_size_t,
                                         ctypes.POINTER(ctypes.c_size_t)]
    lib.orc_allreduce_chunks.restype = None
    lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_bf16.restype = ctypes.c_uint16
    lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_f32.restype = ctypes.c_float
    lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_f16.restype = ctypes.c_uint16
    lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_f32.restype = ctypes.c_float
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    lib.orc_set_num_threads.restype = None
    return lib


def _ptrs(arrays):
    arr = (ctypes.c_void_p * max(1, len(arrays)))()
    for i, a in enumerate(arrays):
        arr[i] = a.ctypes.data
    return arr


def _check_inputs(xs, dtype, count):
    want = NP_DTYPE[dtype]
    for a in xs:
        if a.dtype != want or not a.flags.c_contiguous or a.ndim != 1 or a.size != count:
            raise ValueError("oracle input must be a contiguous 1-D %s array of %d elements"
                             % (np.dtype(want).name, count))


def _call(rc):
    if rc != 0:
        raise RuntimeError("oracle call failed with code %d" % rc)


def num_threads() -> int:
    """OpenMP threads the oracle's element loops use."""
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the following oracle calls (every element keeps its hop
    order, so results are identical at any thread count)."""
    _load().orc_set_num_threads(int(n))


def allreduce_chunks(dtype: str, n: int, count: int) -> list[int]:
    """All-reduce chunk bounds [off_0 .. off_n] (16-byte units, clamped)."""
    out = (ctypes.c_size_t * (n + 1))()
    _load().orc_allreduce_chunks(DTYPE_CODE[dtype], n, count, out)
    return [int(v) for v in out]


def split_p(n: int) -> int:
    """The split avg's pre-scale divisor p (2^e, e the least with 4^e >= n)."""
    return int(_load().orc_split_p(n))


def ring_allreduce(xs, dtype: str, op: str, out=None, counters: bool = False, acc32: bool = False,
                   avg_split: bool = False):
    """Ring all-reduce of the rank buffers ``xs`` (list of n 1-D arrays).

    Returns the list of n outputs (``out`` if given; ``out is xs`` is the
    in-place call), plus ``(hops_per_chunk, bytes_sent_per_rank)`` when
    ``counters`` is true.  ``acc32``: bf16/fp16 partials stay fp32 between
    hops, rounded once at the end; ``avg_split``: float avg pre-scales by
    1/p and divides the finished sum by n/p (``split_p``).
    """
    n = len(xs)
    count = xs[0].size if n else 0
    _check_inputs(xs, dtype, count)
    ys = out if out is not None else [np.empty(count, NP_DTYPE[dtype]) for _ in range(n)]
    _check_inputs(ys, dtype, count)
    hops = (ctypes.c_longlong * max(1, n))()
    sent = (ctypes.c_longlong * max(1, n))()
    _call(_load().orc_ring_allreduce_ex(DTYPE_CODE[dtype], OP_CODE[op], n, count,
                                        _ptrs(xs), _ptrs(ys), hops, sent, int(acc32), int(avg_split)))
    if counters:
        return ys, list(hops)[:n], list(sent)[:n]
    return ys


def ring_reduce_scatter(xs, dtype: str, op: str, out=None, counters: bool = False, acc32: bool = False,
                        avg_split: bool = False):
    """Ring reduce-scatter: each x_r has n*R elements; rank r gets slice r (R elements)."""
    n = len(xs)
    total = xs[0].size
    if total % n:
        raise ValueError("reduce-scatter input size must be a multiple of n")
    R = total // n
    _check_inputs(xs, dtype, total)
    ys = out if out is not None else [np.empty(R, NP_DTYPE[dtype]) for _ in range(n)]
    _check_inputs(ys, dtype, R)
    hops = (ctypes.c_longlong * n)()
    sent = (ctypes.c_longlong * n)()
    _call(_load().orc_ring_reduce_scatter_ex(DTYPE_CODE[dtype], OP_CODE[op], n, R,
                                             _ptrs(xs), _ptrs(ys), hops, sent, int(acc32), int(avg_split)))
    if counters:
        return ys, list(hops), list(sent)
    return ys


def ring_all_gather(xs, dtype: str, out=None, counters: bool = False):
    """Ring all-gather: each x_r has R elements; every rank gets x_0 || ... || x_{n-1}."""
    n = len(xs)
    R = xs[0].size
    _check_inputs(xs, dtype, R)
    ys = out if out is not None else [np.empty(n * R, NP_DTYPE[dtype]) for _ in range(n)]
    _check_inputs(ys, dtype, n * R)
    hops = (ctypes.c_longlong * n)()
    sent = (ctypes.c_longlong * n)()
    _call(_load().orc_ring_all_gather(DTYPE_CODE[dtype], n, R, _ptrs(xs), _ptrs(ys), hops, sent))
    if counters:
        return ys, list(hops), list(sent)
    return ys


def direct_reduce(xs, dtype: str, op: str):
    """The plain definition x_0 (+) ... (+) x_{n-1} (then the avg rule), one
    output array.  Exact for every schedule when dtype is i32 or op is
    min/max; works on any slice of the rank buffers."""
    n = len(xs)
    count = xs[0].size
    _check_inputs(xs, dtype, count)
    y = np.empty(count, NP_DTYPE[dtype])
    _call(_load().orc_direct_reduce(DTYPE_CODE[dtype], OP_CODE[op], n, count, _ptrs(xs), y.ctypes.data))
    return y


def pairwise_reduce(xs, dtype: str, op: str, acc32: bool = False, avg_split: bool = False):
    """All ranks combined at once in the aligned pairwise order over rank
    indices ([lo, lo+len) = [lo, lo+h) (+) [lo+h, lo+len), h the largest power
    of two below len), each combine rounded to the storage type; then the avg
    rule.  One output array (every rank receives it); works on any slice."""
    n = len(xs)
    count = xs[0].size
    _check_inputs(xs, dtype, count)
    y = np.empty(count, NP_DTYPE[dtype])
    _call(_load().orc_pairwise_reduce_ex(DTYPE_CODE[dtype], OP_CODE[op], n, count, _ptrs(xs), y.ctypes.data,
                                         int(acc32), int(avg_split)))
    return y


def tree_parent(n: int, v: int) -> int:
    """Parent of rank v in the bit-trick tree over n ranks (-1 for the root 0)."""
    return int(_load().orc_tree_parent(n, v))


def tree_allreduce(xs, dtype: str, op: str, out=None, acc32: bool = False, avg_split: bool = False):
    """Tree all-reduce: reduce up to rank 0 (own first, children ascending), broadcast down."""
    n = len(xs)
    count = xs[0].size
    _check_inputs(xs, dtype, count)
    ys = out if out is not None else [np.empty(count, NP_DTYPE[dtype]) for _ in range(n)]
    _check_inputs(ys, dtype, count)
    _call(_load().orc_tree_allreduce_ex(DTYPE_CODE[dtype], OP_CODE[op], n, count, _ptrs(xs), _ptrs(ys),
                                        int(acc32), int(avg_split)))
    return ys


def dtree_parent(n: int, which: int, v: int) -> int:
    """Parent of rank v in tree ``which`` (0: the bit-trick tree; 1: its mirror
    for even n, its +1 shift for odd n) of the double binary tree; -1 for a root."""
    return int(_load().orc_dtree_parent(n, which, v))


def dtree_allreduce(xs, dtype: str, op: str, out=None, acc32: bool = False, avg_split: bool = False):
    """Double binary tree all-reduce: elements [0, u*floor(V/2)) up the first
    tree, the rest up the second (u = 16 / element size, V = ceil(count / u))."""
    n = len(xs)
    count = xs[0].size
    _check_inputs(xs, dtype, count)
    ys = out if out is not None else [np.empty(count, NP_DTYPE[dtype]) for _ in range(n)]
    _check_inputs(ys, dtype, count)
    _call(_load().orc_dtree_allreduce_ex(DTYPE_CODE[dtype], OP_CODE[op], n, count, _ptrs(xs), _ptrs(ys),
                                         int(acc32), int(avg_split)))
    return ys


# scalar conversions (exposed for the pins of the oracle's own rounding code)
def f32_to_bf16_bits(v: float) -> int:
    return int(_load().orc_f32_to_bf16(v))


def bf16_bits_to_f32(h: int) -> float:
    return float(_load().orc_bf16_to_f32(h))


def f32_to_f16_bits(v: float) -> int:
    return int(_load().orc_f32_to_f16(v))


def f16_bits_to_f32(h: int) -> float:
    return float(_load().orc_f16_to_f32(h))
