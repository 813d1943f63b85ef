"""Pins of the M-to-N reshard oracle (``oracle.reshard``) against what the
NCCL M2N paper fixes: the ownership tables and schedules it prints
(``tests/golden/m2n_examples.json``), its Eq. (1)/(2) on hand-evaluated cases,
and invariants that hold for any layout (a global tensor whose elements are
their own index must arrive at every destination element's global index;
each destination shard is covered exactly once by its incoming boxes; a
reshard and its inverse compose to the identity)."""
from __future__ import annotations

import itertools
import json
import os

import numpy as np
import pytest

from oracle import reshard as m2n

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "m2n_examples.json")


def golden(name):
    with open(GOLDEN) as f:
        return json.load(f)[name]


def layout(g, side):
    d = g[side]
    return m2n.Layout(tuple(g["shape"]), tuple(d["mesh"]), tuple(d["placements"]), d["base_rank"])


def boxes(b):
    return [list(x) for x in b]


def test_eq1_mesh_rank():
    # Eq. (1): rank(i0, i1) = r0 + i0 * D1 + i1, for a 3 x 5 mesh at base 7
    L = m2n.Layout((6, 10), (3, 5), (-1, 1), 7)
    for i0 in range(3):
        for i1 in range(5):
            slot = i0 * 5 + i1
            assert m2n.mesh_coords(L, slot) == (i0, i1)
            assert m2n.comm_rank(L, slot) == 7 + i0 * 5 + i1


def test_eq2_bounds_hand_evaluated():
    # Eq. (2) with an uneven split: S = 10 over D = 4 gives floor(i*10/4) = 0, 2, 5, 7, 10
    L = m2n.Layout((10,), (4,), (0,))
    assert [m2n.shard_bounds(L, s)[0] for s in range(4)] == [(0, 2), (2, 5), (5, 7), (7, 10)]
    # a replicated dimension spans its full extent; the sharded one its slice
    L = m2n.Layout((6, 9), (2, 3), (-1, 1))
    assert m2n.shard_bounds(L, 4) == [(0, 6), (3, 6)]          # coords (1, 1)
    # a sharded dimension along the first mesh axis
    L = m2n.Layout((6, 9), (2, 3), (0, -1))
    assert m2n.shard_bounds(L, 4) == [(3, 6), (0, 9)]


@pytest.mark.parametrize("S,D", [(8, 4), (10, 4), (7, 7), (5, 8), (1000, 7)])
def test_eq2_bounds_partition_the_dimension(S, D):
    L = m2n.Layout((S,), (D,), (0,))
    b = [m2n.shard_bounds(L, s)[0] for s in range(D)]
    assert b[0][0] == 0 and b[-1][1] == S
    assert all(b[i][1] == b[i + 1][0] for i in range(D - 1))
    sizes = [h - l for l, h in b]
    assert max(sizes) - min(sizes) <= 1
    if S % D == 0:
        assert b == [(i * S // D, (i + 1) * S // D) for i in range(D)]


def test_table3_example_a_ownership():
    g = golden("example_a")
    src, dst = layout(g, "src"), layout(g, "dst")
    got = {}
    for L in (src, dst):
        for s in range(L.size):
            got[str(m2n.comm_rank(L, s))] = boxes(m2n.shard_bounds(L, s))
    assert got == {k: boxes(v) for k, v in g["ownership"].items()}


def test_example_a_schedule_and_flat_volume():
    g = golden("example_a")
    src, dst = layout(g, "src"), layout(g, "dst")
    got = sorted((s, t, boxes(b)) for s, t, b in m2n.plan(src, dst))
    want = sorted((s, t, boxes(b)) for s, t, b in g["transfers"])
    assert got == want
    assert m2n.flat_bytes(src, dst, 4) == g["flat_copies_of_payload"] * m2n.unique_bytes(dst, 4)


def test_table4_example_b_two_calls():
    g = golden("example_b")
    src, dst = layout(g, "src"), layout(g, "dst")
    own = {str(m2n.comm_rank(L, s)): boxes(m2n.shard_bounds(L, s)) for L in (src, dst) for s in range(L.size)}
    assert own == {k: boxes(v) for k, v in g["ownership_by_comm_rank"].items()}
    # two calls (one per PP stage) leave the generator holding one full tensor per stage
    rng = np.random.default_rng(0)
    for stage in range(2):
        full = rng.standard_normal(g["shape"]).astype(np.float32)
        out = m2n.reshard(src, m2n.scatter(src, full), dst)
        assert len(out) == 1 and np.array_equal(out[0].reshape(full.shape), full)


def test_figure3_leader_assignment():
    g = golden("figure3")
    src, dst = layout(g, "src"), layout(g, "dst")
    shards = m2n.dst_shards(dst)
    assert len(shards) == g["K"]
    rho = len(shards[0][1]) // g["domains"]
    assert rho == g["rho"]
    for j, (bounds, _) in enumerate(shards):
        q = sum(1 for s in m2n.owners(src) if m2n.overlap(m2n.shard_bounds(src, s), bounds) is not None)
        assert q == g["q"][j] and divmod(q, rho) == (g["a"][j], g["b"][j])
    lead = m2n.leaders(src, dst, domains=g["domains"])
    got = {str(s): t for (s, j), t in lead.items()}
    assert got == {k: v for k, v in g["leader_of_source"].items()}


@pytest.mark.parametrize("q,rho", [(16, 2), (16, 3), (5, 8), (7, 4), (1, 1), (9, 9)])
def test_leader_loads_differ_by_at_most_one(q, rho):
    # q source shards along dim 0, one destination shard replicated rho times
    src = m2n.Layout((q * 2, 3), (q,), (0,))
    dst = m2n.Layout((q * 2, 3), (rho,), (-1,))
    lead = m2n.leaders(src, dst)
    assert len(lead) == q                                      # every contribution enters exactly once
    loads = [list(lead.values()).count(m2n.comm_rank(dst, i)) for i in range(rho)]
    assert max(loads) - min(loads) <= 1 and sum(loads) == q
    a, b = divmod(q, rho)
    assert loads == [a + 1] * b + [a] * (rho - b)              # the first q mod rho take one more
    # ordered by source shard: contributions go to replicas in runs
    order = [lead[(s, 0)] for s in range(q)]
    assert order == sorted(order)


def test_moe_layer_workload_counts():
    g = golden("moe_layer")
    S = tuple(g["shape"])
    for dp in g["trainer_dp"]:
        src = m2n.Layout(S, (dp, g["active_sources"]), (-1, 0))
        assert len(m2n.owners(src)) == g["active_sources"]      # replicas collapse to one owner
        for rd in g["r_d"]:
            dst = m2n.Layout(S, (rd, g["K"]), (-1, 1), src.size)
            assert m2n.unique_bytes(dst, g["elem_size"]) == g["unique_mib"] << 20
            assert len(m2n.dst_shards(dst)) == g["K"]
            tr = m2n.plan(src, dst)
            assert len(tr) == g["active_sources"] * g["K"] * rd
            assert m2n.flat_bytes(src, dst, g["elem_size"]) == rd * (g["unique_mib"] << 20)
            loads = {}
            for _, t in m2n.leaders(src, dst).items():
                loads[t] = loads.get(t, 0) + 1
            assert sorted(set(loads.values())) == [g["active_sources"] // rd]


def _random_layout(rng, shape, nranks_max=6):
    nd_mesh = int(rng.integers(1, 3))
    mesh = tuple(int(rng.integers(1, 4)) for _ in range(nd_mesh))
    placements = [-1] * nd_mesh
    k = int(rng.integers(0, nd_mesh + 1))                      # at most one sharded axis (k == nd_mesh: none)
    if k < nd_mesh:
        placements[k] = int(rng.integers(0, len(shape)))
    return m2n.Layout(tuple(shape), mesh, tuple(placements), int(rng.integers(0, 5)))


def _layout_pairs(seed, count):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        nd = int(rng.integers(1, 4))
        shape = tuple(int(rng.integers(1, 7)) for _ in range(nd))
        yield _random_layout(rng, shape), _random_layout(rng, shape)


def test_identity_tensor_reaches_every_global_index():
    """Brute force: the global tensor holds each element's own linear index;
    every destination element must hold the linear index of its global
    position (local index + the shard's lower bounds, Eq. (2))."""
    for src, dst in _layout_pairs(1, 300):
        full = np.arange(int(np.prod(src.shape)), dtype=np.int64).reshape(src.shape)
        out = m2n.reshard(src, m2n.scatter(src, full), dst)
        for t in range(dst.size):
            b = m2n.shard_bounds(dst, t)
            ext = [h - l for l, h in b]
            assert out[t].size == int(np.prod(ext))
            for flat, local in enumerate(itertools.product(*[range(e) for e in ext])):
                gidx = 0
                for d, (x, (l, _)) in enumerate(zip(local, b)):
                    gidx = gidx * src.shape[d] + (l + x)
                assert out[t][flat] == gidx


def test_incoming_boxes_tile_each_destination_exactly_once():
    for src, dst in _layout_pairs(2, 300):
        tr = m2n.plan(src, dst)
        for t in range(dst.size):
            rank = m2n.comm_rank(dst, t)
            b = m2n.shard_bounds(dst, t)
            cover = np.zeros([h - l for l, h in b], dtype=np.int32)
            for _, tt, box in tr:
                if tt == rank:
                    cover[tuple(slice(lo - l, hi - l) for (lo, hi), (l, _) in zip(box, b))] += 1
            assert (cover == 1).all()
        # sources in the plan are the owners only (replicas collapsed, lowest slot)
        own = {m2n.comm_rank(src, s) for s in m2n.owners(src)}
        assert {s for s, _, _ in tr} <= own


def test_replicated_sources_collapse_to_the_lowest_slot():
    src = m2n.Layout((4, 6), (3, 2), (-1, 1), 10)              # 3 replicas of 2 shards
    assert m2n.owners(src) == [0, 1]
    dst = m2n.Layout((4, 6), (2,), (0,), 0)
    assert {s for s, _, _ in m2n.plan(src, dst)} == {10, 11}


def test_round_trip_is_the_identity():
    rng = np.random.default_rng(3)
    for src, dst in _layout_pairs(4, 100):
        full = rng.standard_normal(src.shape).astype(np.float32)
        mid = m2n.reshard(src, m2n.scatter(src, full), dst)
        back = m2n.reshard(dst, mid, src)
        for s, want in enumerate(m2n.scatter(src, full)):
            assert np.array_equal(back[s], want)


def test_mismatched_global_shapes_are_rejected():
    with pytest.raises(AssertionError):
        m2n.reshard(m2n.Layout((4, 8), (2,), (0,)), [np.zeros(16, np.float32)] * 2, m2n.Layout((8, 4), (1,), (-1,)))
