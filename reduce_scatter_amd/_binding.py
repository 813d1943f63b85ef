"""ctypes marshalling for libar.so (see ``include/ar.h`` for the contract).

Buffers may be given as torch tensors (their ``data_ptr()`` is used) or as
integer device addresses.  ``stream`` may be a ``torch.cuda.Stream``, an
integer ``hipStream_t`` handle, or None for torch's current stream on the
current device (the NULL stream when torch is absent).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libar.so")

AR_MAX_RANKS = 128
DTYPES = {"f32": 0, "bf16": 1, "f16": 2, "i32": 3}
OPS = {"sum": 0, "prod": 1, "min": 2, "max": 3, "avg": 4}
SCHEDS = {"auto": 0, "ring": 1, "tree": 2, "fused": 3, "split": 4, "dtree": 5}
COLLS = {"allreduce": 0, "reduce_scatter": 1, "all_gather": 2}
ACCS = {"storage": 0, "fp32": 1}
AVGS = {"prescale": 0, "split": 1}
_SCHED_NAMES = {v: k for k, v in SCHEDS.items()}
_STATUS = {0: "AR_OK", 1: "AR_ERR_INVALID_ARG", 2: "AR_ERR_UNSUPPORTED", 3: "AR_ERR_ALIGNMENT", 4: "AR_ERR_HIP"}

if not os.path.exists(_LIB_PATH):
    raise ImportError("libar.so is not built (expected at %s); build it with `python reduce_scatter_amd/build.py` "
                      "or __graft_entry__.build()" % _LIB_PATH)

# One HIP runtime per process: PyTorch-ROCm ships its own libamdhip64 (same
# SONAME as the system one).  Loading torch first makes libar.so bind to the
# runtime torch already loaded; loading libar.so first would pull in the
# system copy and torch would then load a second, separate runtime, whose
# devices, streams and allocations are not the ones libar.so sees.
try:
    import torch  # noqa: F401
except ImportError:
    pass

_lib = ctypes.CDLL(_LIB_PATH)


class _Numerics(ctypes.Structure):
    _fields_ = [("acc", ctypes.c_int), ("avg", ctypes.c_int)]


class _PlanStruct(ctypes.Structure):
    _fields_ = [("chosen", ctypes.c_int), ("legal_mask", ctypes.c_uint), ("steps", ctypes.c_int * 6),
                ("bytes", ctypes.c_double * 6), ("predicted_us", ctypes.c_double * 6)]


_vpp = ctypes.POINTER(ctypes.c_void_p)
_lib.ar_allreduce.argtypes = [_vpp, _vpp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                              ctypes.c_void_p]
_lib.ar_reduce_scatter.argtypes = _lib.ar_allreduce.argtypes
_lib.ar_allreduce_ex.argtypes = [_vpp, _vpp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
_lib.ar_reduce_scatter_ex.argtypes = _lib.ar_allreduce_ex.argtypes
_lib.ar_all_gather.argtypes = [_vpp, _vpp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_void_p]
_lib.ar_plan.argtypes = [ctypes.c_int, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                         ctypes.POINTER(_PlanStruct)]
_lib.ar_tree_parent.argtypes = [ctypes.c_int, ctypes.c_int]
_lib.ar_tree_parent.restype = ctypes.c_int
_lib.ar_dtree_parent.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
_lib.ar_dtree_parent.restype = ctypes.c_int
_lib.ar_status_string.argtypes = [ctypes.c_int]
_lib.ar_status_string.restype = ctypes.c_char_p
for _f in (_lib.ar_allreduce, _lib.ar_reduce_scatter, _lib.ar_all_gather, _lib.ar_plan, _lib.ar_allreduce_ex,
           _lib.ar_reduce_scatter_ex):
    _f.restype = ctypes.c_int


def library_path() -> str:
    return _LIB_PATH


class ArError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        self.name = _STATUS.get(status, str(status))
        super().__init__(ar_status_string(status))


@dataclass
class Plan:
    chosen: str
    legal: list
    steps: dict
    bytes: dict
    predicted_us: dict


def ar_status_string(status: int) -> str:
    return _lib.ar_status_string(int(status)).decode()


def _code(table, value, what):
    if isinstance(value, str):
        if value not in table:
            raise ValueError("unknown %s %r (expected one of %s)" % (what, value, sorted(table)))
        return table[value]
    return int(value)


def _dtype_code(dtype):
    try:
        import torch
        tmap = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16", torch.int32: "i32"}
        if dtype in tmap:
            dtype = tmap[dtype]
    except ImportError:
        pass
    return _code(DTYPES, dtype, "dtype")


def _ptr(b):
    if b is None:
        return None
    if isinstance(b, int):
        return b
    return int(b.data_ptr())


class PointerTable:
    """A host array of device pointers built once and reusable across calls
    (a list of tensors costs a ``data_ptr()`` call per buffer on every call;
    at 128 ranks that host time is comparable to a small collective).  The
    table keeps references to the tensors it was built from."""

    def __init__(self, bufs):
        self.n = len(bufs)
        self.array = (ctypes.c_void_p * max(1, self.n))(*[_ptr(b) for b in bufs])
        self._bufs = list(bufs)          # tensors stay alive (and their memory owned) while the table exists

    def __len__(self):
        return self.n


def pointers(bufs) -> PointerTable:
    """Build a reusable pointer table for ``bufs`` (tensors or integer addresses)."""
    return PointerTable(bufs)


def _ptr_array(bufs):
    if isinstance(bufs, PointerTable):
        return bufs.array
    return (ctypes.c_void_p * max(1, len(bufs)))(*[_ptr(b) for b in bufs])


def _tables(sendbufs, recvbufs):
    send = _ptr_array(sendbufs)
    return send, (send if recvbufs is sendbufs else _ptr_array(recvbufs))


_gpu_state = []     # [current-stream getter] once known; [None] without torch or a GPU


def _current_stream_getter():
    try:
        import torch
    except ImportError:
        return None
    if not torch.cuda.is_available():
        return None
    raw, dev = getattr(torch._C, "_cuda_getCurrentRawStream", None), getattr(torch._C, "_cuda_getDevice", None)
    if raw is not None and dev is not None:
        return lambda: raw(dev())                      # the handle of torch's current stream, without a Stream object
    return lambda: int(torch.cuda.current_stream().cuda_stream)


def _stream(stream):
    if stream is None:
        if not _gpu_state:
            _gpu_state.append(_current_stream_getter())
        get = _gpu_state[0]
        return get() if get is not None else 0
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(status):
    if status != 0:
        raise ArError(status)


def ar_allreduce(sendbufs, recvbufs, count, dtype, op, n=None, sched="auto", stream=None):
    """All-reduce ``count`` elements of each of the n rank buffers (in place when recvbufs is sendbufs)."""
    n = len(sendbufs) if n is None else n
    send, recv = _tables(sendbufs, recvbufs)
    _check(_lib.ar_allreduce(send, recv, count, _dtype_code(dtype),
                             _code(OPS, op, "op"), n, _code(SCHEDS, sched, "schedule"), _stream(stream)))


def ar_reduce_scatter(sendbufs, recvbufs, recvcount, dtype, op, n=None, sched="auto", stream=None):
    """Reduce-scatter: each send buffer holds n*recvcount elements; rank r receives slice r."""
    n = len(sendbufs) if n is None else n
    send, recv = _tables(sendbufs, recvbufs)
    _check(_lib.ar_reduce_scatter(send, recv, recvcount, _dtype_code(dtype),
                                  _code(OPS, op, "op"), n, _code(SCHEDS, sched, "schedule"), _stream(stream)))


def _numerics(acc, avg):
    return ctypes.byref(_Numerics(_code(ACCS, acc, "accumulation"), _code(AVGS, avg, "avg route")))


def ar_allreduce_ex(sendbufs, recvbufs, count, dtype, op, n=None, sched="auto", acc="storage", avg="prescale",
                    stream=None):
    """All-reduce with explicit numerics: ``acc`` "storage" | "fp32" (bf16 / fp16
    partials kept in fp32, fused schedule), ``avg`` "prescale" | "split"."""
    n = len(sendbufs) if n is None else n
    send, recv = _tables(sendbufs, recvbufs)
    _check(_lib.ar_allreduce_ex(send, recv, count, _dtype_code(dtype), _code(OPS, op, "op"), n,
                                _code(SCHEDS, sched, "schedule"), _numerics(acc, avg), _stream(stream)))


def ar_reduce_scatter_ex(sendbufs, recvbufs, recvcount, dtype, op, n=None, sched="auto", acc="storage",
                         avg="prescale", stream=None):
    """Reduce-scatter with explicit numerics (as :func:`ar_allreduce_ex`)."""
    n = len(sendbufs) if n is None else n
    send, recv = _tables(sendbufs, recvbufs)
    _check(_lib.ar_reduce_scatter_ex(send, recv, recvcount, _dtype_code(dtype), _code(OPS, op, "op"), n,
                                     _code(SCHEDS, sched, "schedule"), _numerics(acc, avg), _stream(stream)))


def ar_all_gather(sendbufs, recvbufs, sendcount, dtype, n=None, sched="auto", stream=None):
    """All-gather: each rank receives the n pieces of sendcount elements, in rank order."""
    n = len(sendbufs) if n is None else n
    send, recv = _tables(sendbufs, recvbufs)
    _check(_lib.ar_all_gather(send, recv, sendcount, _dtype_code(dtype), n,
                              _code(SCHEDS, sched, "schedule"), _stream(stream)))


def ar_plan(coll, count, dtype, op, n) -> Plan:
    """The cost model's choice for a call (host only; no GPU needed)."""
    p = _PlanStruct()
    _check(_lib.ar_plan(_code(COLLS, coll, "collective"), count, _dtype_code(dtype), _code(OPS, op, "op"), n,
                        ctypes.byref(p)))
    legal = [name for name, s in SCHEDS.items() if s and (p.legal_mask >> s) & 1]
    return Plan(chosen=_SCHED_NAMES[p.chosen], legal=legal,
                steps={s: p.steps[SCHEDS[s]] for s in legal},
                bytes={s: p.bytes[SCHEDS[s]] for s in legal},
                predicted_us={s: p.predicted_us[SCHEDS[s]] for s in legal})


def ar_tree_parent(n: int, v: int) -> int:
    return int(_lib.ar_tree_parent(n, v))


def ar_dtree_parent(n: int, which: int, v: int) -> int:
    return int(_lib.ar_dtree_parent(n, which, v))


# ---------------------------------------------------------------------------
# M-to-N layout reshard (include/ar_reshard.h)
# ---------------------------------------------------------------------------

REPLICATE = -1
ROUTES = {"auto": 0, "flat": 1, "hier": 2, "fused": 3}
_ROUTE_NAMES = {v: k for k, v in ROUTES.items()}


class _Layout(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int), ("shape", ctypes.c_longlong * 3), ("mesh_ndim", ctypes.c_int),
                ("mesh", ctypes.c_int * 2), ("placement", ctypes.c_int * 2), ("base_rank", ctypes.c_int)]


class _Transfer(ctypes.Structure):
    _fields_ = [("src_rank", ctypes.c_int), ("dst_rank", ctypes.c_int), ("leader_rank", ctypes.c_int),
                ("lo", ctypes.c_longlong * 3), ("hi", ctypes.c_longlong * 3), ("bytes", ctypes.c_longlong)]


class _ReshardPlanStruct(ctypes.Structure):
    _fields_ = [("chosen", ctypes.c_int), ("n_transfers", ctypes.c_int), ("n_sources", ctypes.c_int),
                ("n_shards", ctypes.c_int), ("max_replicas", ctypes.c_int), ("unique_bytes", ctypes.c_longlong),
                ("bytes", ctypes.c_double * 4), ("launches", ctypes.c_int * 4), ("predicted_us", ctypes.c_double * 4)]


_lib.ar_reshard_plan.argtypes = [ctypes.POINTER(_Layout), ctypes.POINTER(_Layout), ctypes.c_size_t, ctypes.c_int,
                                 ctypes.POINTER(_ReshardPlanStruct), ctypes.POINTER(_Transfer), ctypes.c_int]
_lib.ar_reshard_plan.restype = ctypes.c_int
_lib.ar_reshard.argtypes = [_vpp, _vpp, ctypes.POINTER(_Layout), ctypes.POINTER(_Layout), ctypes.c_size_t,
                            ctypes.c_int, ctypes.c_void_p]
_lib.ar_reshard.restype = ctypes.c_int


@dataclass(frozen=True)
class Layout:
    """An endpoint layout (S, M, p): global ``shape``, ``mesh`` extents, one
    placement per mesh axis (REPLICATE or the sharded tensor dimension) and
    the mesh's ``base_rank``."""
    shape: tuple
    mesh: tuple
    placements: tuple
    base_rank: int = 0


_lib.ar_layout_shard.argtypes = [ctypes.POINTER(_Layout), ctypes.c_int, ctypes.POINTER(ctypes.c_longlong),
                                 ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(ctypes.c_int)]
_lib.ar_layout_shard.restype = ctypes.c_int


def _layout(L):
    """Any object with ``shape``, ``mesh``, ``placements`` (REPLICATE or the
    sharded tensor dimension per mesh axis) and optionally ``base_rank``."""
    s = _Layout()
    shape, mesh, pl = tuple(L.shape), tuple(L.mesh), tuple(L.placements)
    if not (1 <= len(shape) <= 3 and 1 <= len(mesh) <= 2 and len(pl) == len(mesh)):
        raise ValueError("a layout has 1-3 tensor dimensions and 1-2 mesh axes, one placement per axis")
    s.ndim, s.mesh_ndim = len(shape), len(mesh)
    for d, v in enumerate(shape):
        s.shape[d] = int(v)
    for k in range(len(mesh)):
        s.mesh[k] = int(mesh[k])
        s.placement[k] = int(pl[k])
    s.base_rank = int(getattr(L, "base_rank", 0))
    return s


def ar_layout_shard(layout, slot):
    """([(lo, hi)] per tensor dimension, communicator rank) of mesh slot ``slot``."""
    L = _layout(layout)
    lo, hi, rank = (ctypes.c_longlong * 3)(), (ctypes.c_longlong * 3)(), ctypes.c_int()
    _check(_lib.ar_layout_shard(ctypes.byref(L), slot, lo, hi, ctypes.byref(rank)))
    return [(lo[d], hi[d]) for d in range(L.ndim)], rank.value


def local_shape(layout, slot):
    """Shape of mesh slot ``slot``'s local buffer."""
    return tuple(h - l for l, h in ar_layout_shard(layout, slot)[0])


@dataclass
class ReshardPlan:
    chosen: str
    n_transfers: int
    n_sources: int
    n_shards: int
    max_replicas: int
    unique_bytes: int
    bytes: dict
    launches: dict
    predicted_us: dict
    transfers: list        # (src_rank, dst_rank, leader_rank, [(lo, hi)] per tensor dim, bytes)


def ar_reshard_plan(src, dst, elem_size, domains=1) -> ReshardPlan:
    """The layout-derived schedule and route costs (host only)."""
    ls, ld = _layout(src), _layout(dst)
    out = _ReshardPlanStruct()
    _check(_lib.ar_reshard_plan(ctypes.byref(ls), ctypes.byref(ld), elem_size, domains, ctypes.byref(out), None, 0))
    n = out.n_transfers
    arr = (_Transfer * max(1, n))()
    _check(_lib.ar_reshard_plan(ctypes.byref(ls), ctypes.byref(ld), elem_size, domains, ctypes.byref(out), arr, n))
    nd = ls.ndim
    transfers = [(t.src_rank, t.dst_rank, t.leader_rank, [(t.lo[d], t.hi[d]) for d in range(nd)], t.bytes)
                 for t in arr[:n]]
    names = ("flat", "hier", "fused")
    return ReshardPlan(_ROUTE_NAMES[out.chosen], n, out.n_sources, out.n_shards, out.max_replicas,
                       out.unique_bytes, {k: out.bytes[ROUTES[k]] for k in names},
                       {k: out.launches[ROUTES[k]] for k in names},
                       {k: out.predicted_us[ROUTES[k]] for k in names}, transfers)


def ar_reshard(src_bufs, dst_bufs, src, dst, elem_size, route="auto", stream=None):
    """Reshard from layout ``src`` (buffers ``src_bufs``, one per source mesh
    slot; None allowed for replicas that are not the owner of their shard)
    to layout ``dst`` (``dst_bufs``, one per destination slot)."""
    ls, ld = _layout(src), _layout(dst)
    _check(_lib.ar_reshard(_ptr_array(src_bufs), _ptr_array(dst_bufs), ctypes.byref(ls), ctypes.byref(ld),
                           elem_size, _code(ROUTES, route, "route"), _stream(stream)))
