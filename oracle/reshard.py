"""CPU oracle for the M-to-N layout reshard -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the product library never does, and
nothing here comes from the product (the two share no code).

Everything follows the "NCCL M2N" paper ("NCCL M2N: A Layout- and
Topology-Aware Collective for Distributed Tensor Resharding",
arxiv.org/html/2610.07516):

* §IV "Reshard Semantics and Descriptors": a layout is (S, M, p), a global
  shape, a process mesh and one placement per mesh axis (``Shard(d)`` or
  ``Replicate``); mesh slots map to communicator ranks row-major from a base
  rank (Eq. (1)); a rank's local shard along tensor dimension d is
  [floor(i_k S_d / D_k), floor((i_k+1) S_d / D_k)) when mesh axis k shards d,
  the full extent otherwise (Eq. (2)); a reshard leaves every destination
  rank holding the local shard its layout prescribes.  :func:`mesh_coords`,
  :func:`comm_rank`, :func:`shard_bounds`, :func:`reshard`.
* §V-A "Deterministic Schedule Derivation": for every (source, destination)
  pair the per-dimension overlap [max(l), min(u)); pairs with an empty
  overlap are skipped; replicated source copies collapse to one owner.
  :func:`plan`.
* §V-B "Hierarchical Topology Route": per destination shard j with q_j unique
  contributions and rho local replicas, ordered by source shard, every
  replica gets floor(q_j / rho) and the first q_j mod rho one more; replicas
  with a nonzero load are leaders.  :func:`leaders`.

Readings where the paper leaves a step open:

* the one owner of a replicated source shard is its lowest mesh slot (the
  paper says only "one deterministic owner");
* a destination shard's replicas are its slots in mesh-slot order; with d
  destination domains the first rho = r / d of them form the first domain,
  which holds the leaders;
* local buffers are the row-major local shard, contiguous.

A tensor is a numpy array of any element type; the reshard only moves
elements, so every comparison is exact.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

REPLICATE = -1


def Shard(d: int) -> int:          # noqa: N802  (the paper's placement name)
    """Placement: the mesh axis partitions tensor dimension ``d``."""
    return int(d)


@dataclass(frozen=True)
class Layout:
    """(S, M, p) of §IV: ``shape`` = S, ``mesh`` = (D_0, ...), ``placements``
    = one entry per mesh axis, ``REPLICATE`` or the sharded tensor dimension;
    ``base_rank`` = r_0 of Eq. (1)."""
    shape: tuple
    mesh: tuple
    placements: tuple
    base_rank: int = 0

    @property
    def size(self) -> int:
        return int(np.prod(self.mesh))


def mesh_coords(layout: Layout, slot: int) -> tuple:
    """Mesh coordinates (i_0, i_1, ...) of slot ``slot`` (row-major, Eq. (1))."""
    coords = []
    for D in reversed(layout.mesh):
        coords.append(slot % D)
        slot //= D
    return tuple(reversed(coords))


def comm_rank(layout: Layout, slot: int) -> int:
    """Eq. (1): r_0 + i_0 D_1 + i_1 (row-major over any number of axes)."""
    r = 0
    for i, D in zip(mesh_coords(layout, slot), layout.mesh):
        r = r * D + i
    return layout.base_rank + r


def shard_bounds(layout: Layout, slot: int) -> list:
    """Eq. (2): [(l_d, u_d)] for every tensor dimension d of slot ``slot``."""
    coords = mesh_coords(layout, slot)
    bounds = []
    for d, S in enumerate(layout.shape):
        lo, hi = 0, S
        for k, p in enumerate(layout.placements):
            if p == d:
                lo = (coords[k] * S) // layout.mesh[k]
                hi = ((coords[k] + 1) * S) // layout.mesh[k]
        bounds.append((lo, hi))
    return bounds


def local_shape(layout: Layout, slot: int) -> tuple:
    return tuple(hi - lo for lo, hi in shard_bounds(layout, slot))


def _box(bounds):
    return tuple(slice(lo, hi) for lo, hi in bounds)


def scatter(layout: Layout, full: np.ndarray) -> list:
    """Local shards (flat, row-major) of a global tensor under ``layout``."""
    assert tuple(full.shape) == tuple(layout.shape)
    return [np.ascontiguousarray(full[_box(shard_bounds(layout, s))]).ravel() for s in range(layout.size)]


def reshard(src: Layout, src_bufs: list, dst: Layout) -> list:
    """The reshard's result by its definition (§IV "Reshard"): assemble the
    global tensor from the source shards (replicas must agree), then give
    every destination slot its own shard.  Returns flat row-major buffers,
    one per destination slot."""
    assert tuple(src.shape) == tuple(dst.shape), "both layouts describe one global shape"
    dtype = src_bufs[0].dtype
    full = np.zeros(src.shape, dtype=dtype)
    seen = np.zeros(src.shape, dtype=bool)
    for s in range(src.size):
        box = _box(shard_bounds(src, s))
        piece = np.asarray(src_bufs[s]).reshape(local_shape(src, s))
        prev = seen[box]
        if prev.any():
            assert np.array_equal(full[box][prev], piece[prev]), "replicated source shards disagree"
        full[box] = piece
        seen[box] = True
    assert seen.all(), "the source layout does not cover the tensor"
    return scatter(dst, full)


def owners(layout: Layout) -> list:
    """Slots that own a distinct shard: the lowest slot of every set of
    replicas (the deterministic owner of §V-A)."""
    first = {}
    for s in range(layout.size):
        key = tuple(shard_bounds(layout, s))
        first.setdefault(key, s)
    return sorted(first.values())


def overlap(a: list, b: list):
    """§V-A: per-dimension [max(l), min(u)); None when any is empty."""
    lo = [max(x[0], y[0]) for x, y in zip(a, b)]
    hi = [min(x[1], y[1]) for x, y in zip(a, b)]
    if any(l >= h for l, h in zip(lo, hi)):
        return None
    return list(zip(lo, hi))


def plan(src: Layout, dst: Layout) -> list:
    """§V-A schedule: (source comm rank, destination comm rank, box) for every
    owner source slot (slot order) and destination slot (slot order) whose
    shards overlap; ``box`` = [(lo_d, hi_d)] in global coordinates."""
    out = []
    for s in owners(src):
        bs = shard_bounds(src, s)
        for t in range(dst.size):
            box = overlap(bs, shard_bounds(dst, t))
            if box is not None:
                out.append((comm_rank(src, s), comm_rank(dst, t), box))
    return out


def dst_shards(dst: Layout) -> list:
    """Distinct destination shards j, in order of their first slot, each with
    its replica slots in slot order: [(bounds, [slots])]."""
    groups = {}
    order = []
    for t in range(dst.size):
        key = tuple(shard_bounds(dst, t))
        if key not in groups:
            groups[key] = []
            order.append(key)
        groups[key].append(t)
    return [(list(k), groups[k]) for k in order]


def leaders(src: Layout, dst: Layout, domains: int = 1) -> dict:
    """§V-B leader assignment: {(source comm rank, destination shard index j):
    destination comm rank of the leader replica that receives it}.  With
    ``domains`` destination domains, rho = r / domains replicas of shard j
    (the first rho in slot order) share its q_j contributions, ordered by
    source shard: replica i takes floor(q_j / rho) of them, the first
    q_j mod rho one more."""
    out = {}
    srcs = owners(src)
    for j, (bounds, slots) in enumerate(dst_shards(dst)):
        assert len(slots) % domains == 0, "replicas split evenly over the domains"
        rho = len(slots) // domains
        contrib = [s for s in srcs if overlap(shard_bounds(src, s), bounds) is not None]
        q = len(contrib)
        a, b = divmod(q, rho)
        pos = 0
        for i in range(rho):
            take = a + (1 if i < b else 0)
            for s in contrib[pos:pos + take]:
                out[(comm_rank(src, s), j)] = comm_rank(dst, slots[i])
            pos += take
        assert pos == q
    return out


def flat_bytes(src: Layout, dst: Layout, elem_size: int) -> int:
    """Bytes a flat direct-send realization moves (one copy per transfer)."""
    return sum(int(np.prod([h - l for l, h in box])) for _, _, box in plan(src, dst)) * elem_size


def unique_bytes(dst: Layout, elem_size: int) -> int:
    """B of §V-C: the unique payload, one copy of every destination shard."""
    return sum(int(np.prod([h - l for l, h in b])) for b, _ in dst_shards(dst)) * elem_size
