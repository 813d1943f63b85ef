"""The reshard C ABI without a GPU: the planner's schedule and leaders against
the oracle (exact integers), the printed examples through the ABI, route
volumes, and argument validation (before any HIP call)."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

from oracle import reshard as m2n

ar = pytest.importorskip("reduce_scatter_amd", reason="libar.so not built")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "m2n_examples.json")


def golden(name):
    with open(GOLDEN) as f:
        return json.load(f)[name]


def layout(g, side):
    d = g[side]
    return m2n.Layout(tuple(g["shape"]), tuple(d["mesh"]), tuple(d["placements"]), d["base_rank"])


def random_layout(rng, shape):
    """1-2 mesh axes of 1-4 slots; each axis replicates or shards a tensor
    dimension no other axis shards."""
    nd_mesh = int(rng.integers(1, 3))
    mesh = tuple(int(rng.integers(1, 5)) for _ in range(nd_mesh))
    free = list(range(len(shape)))
    placements = []
    for _ in range(nd_mesh):
        if free and rng.random() < 0.7:
            d = free.pop(int(rng.integers(0, len(free))))
            placements.append(d)
        else:
            placements.append(m2n.REPLICATE)
    return m2n.Layout(tuple(shape), mesh, tuple(placements), int(rng.integers(0, 9)))


def layout_pairs(seed, count, max_extent=9):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        nd = int(rng.integers(1, 4))
        shape = tuple(int(rng.integers(0 if rng.random() < 0.03 else 1, max_extent)) for _ in range(nd))
        yield random_layout(rng, shape), random_layout(rng, shape)


def oracle_transfers(src, dst, domains=1):
    lead = m2n.leaders(src, dst, domains)
    shard_index = {}
    for j, (bounds, slots) in enumerate(m2n.dst_shards(dst)):
        for t in slots:
            shard_index[m2n.comm_rank(dst, t)] = j
    out = []
    for s, t, box in m2n.plan(src, dst):
        out.append((s, t, lead[(s, shard_index[t])], [tuple(b) for b in box]))
    return out


def test_every_declared_function_is_exported():
    import ctypes
    import re
    text = open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "ar_reshard.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(ar_[a-z_]+)\s*\(", text))
    assert names == {"ar_reshard", "ar_reshard_plan", "ar_layout_shard"}
    lib = ctypes.CDLL(ar.library_path())
    for name in names:
        assert hasattr(lib, name), name


def test_layout_shards_match_the_oracle():
    for src, dst in layout_pairs(12, 300):
        for L in (src, dst):
            for s in range(L.size):
                bounds, rank = ar.ar_layout_shard(L, s)
                assert bounds == m2n.shard_bounds(L, s) and rank == m2n.comm_rank(L, s)
                assert ar.local_shape(L, s) == m2n.local_shape(L, s)
    L = m2n.Layout((4, 8), (2,), (0,))
    assert _err(ar.ar_layout_shard, L, 2) == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_layout_shard, L, -1) == "AR_ERR_INVALID_ARG"


def test_plan_matches_the_oracle_on_random_layouts():
    for src, dst in layout_pairs(11, 400):
        p = ar.ar_reshard_plan(src, dst, 4)
        got = [(s, t, lead, [tuple(b) for b in box]) for s, t, lead, box, _ in p.transfers]
        assert got == oracle_transfers(src, dst), (src, dst)
        assert p.n_transfers == len(got)
        assert p.n_sources == len(m2n.owners(src))
        assert p.n_shards == len(m2n.dst_shards(dst))
        assert p.unique_bytes == m2n.unique_bytes(dst, 4)
        for (_, _, _, box, nbytes) in p.transfers:
            assert nbytes == 4 * int(np.prod([h - l for l, h in box]))


def test_plan_leaders_with_domains_match_the_oracle():
    rng = np.random.default_rng(5)
    for _ in range(200):
        shape = (int(rng.integers(1, 12)), int(rng.integers(1, 5)))
        q = int(rng.integers(1, 6))
        src = m2n.Layout(shape, (int(rng.integers(1, 3)), q), (-1, 0), 0)
        domains = int(rng.integers(1, 4))
        rho = int(rng.integers(1, 4))
        K = int(rng.integers(1, 4))
        dst = m2n.Layout(shape, (domains * rho, K), (-1, int(rng.integers(0, 2))), src.size)
        p = ar.ar_reshard_plan(src, dst, 2, domains=domains)
        got = [(s, t, lead, [tuple(b) for b in box]) for s, t, lead, box, _ in p.transfers]
        assert got == oracle_transfers(src, dst, domains)


def test_printed_examples_through_the_abi():
    g = golden("example_a")
    p = ar.ar_reshard_plan(layout(g, "src"), layout(g, "dst"), 4)
    got = sorted((s, t, [list(b) for b in box]) for s, t, _, box, _ in p.transfers)
    assert got == sorted((s, t, box) for s, t, box in g["transfers"])
    assert p.bytes["flat"] == 2 * g["flat_copies_of_payload"] * p.unique_bytes     # read + write per copy
    g = golden("figure3")
    p = ar.ar_reshard_plan(layout(g, "src"), layout(g, "dst"), 4, domains=g["domains"])
    leaders = {str(s): lead for s, _, lead, _, _ in p.transfers}
    assert leaders == g["leader_of_source"]


def test_route_volumes_and_choice():
    g = golden("moe_layer")
    S = tuple(g["shape"])
    B = g["unique_mib"] << 20
    for rd in g["r_d"]:
        src = m2n.Layout(S, (1, g["active_sources"]), (-1, 0))
        dst = m2n.Layout(S, (rd, g["K"]), (-1, 1), src.size)
        p = ar.ar_reshard_plan(src, dst, g["elem_size"])
        assert p.unique_bytes == B
        assert p.n_transfers == g["active_sources"] * g["K"] * rd
        assert p.bytes == {"flat": 2 * rd * B, "hier": (2 + rd) * B, "fused": (1 + rd) * B}
        assert p.chosen == "fused"            # fewest bytes and fewest launches when every replica shares one HBM
        assert p.launches["fused"] <= p.launches["hier"] and p.launches["fused"] <= p.launches["flat"]


def _err(fn, *a, **k):
    try:
        fn(*a, **k)
    except ar.ArError as e:
        return str(e).split(":")[0]
    return "AR_OK"


def test_plan_rejects_bad_layouts():
    ok = m2n.Layout((4, 8), (2,), (0,))
    assert _err(ar.ar_reshard_plan, ok, ok, 4) == "AR_OK"
    assert _err(ar.ar_reshard_plan, ok, m2n.Layout((8, 4), (2,), (0,)), 4) == "AR_ERR_INVALID_ARG"   # shapes differ
    assert _err(ar.ar_reshard_plan, ok, m2n.Layout((4, 8), (2,), (2,)), 4) == "AR_ERR_INVALID_ARG"   # no dim 2
    assert _err(ar.ar_reshard_plan, ok, m2n.Layout((4, 8), (0,), (0,)), 4) == "AR_ERR_INVALID_ARG"   # empty mesh
    assert _err(ar.ar_reshard_plan, ok, m2n.Layout((4, 8), (16, 16), (0, 1)), 4) == "AR_ERR_INVALID_ARG"  # > 128
    assert _err(ar.ar_reshard_plan, ok, m2n.Layout((4, 8), (2, 2), (0, 0)), 4) == "AR_ERR_UNSUPPORTED"   # dim twice
    assert _err(ar.ar_reshard_plan, ok, ok, 3) == "AR_ERR_UNSUPPORTED"                                 # elem size
    assert _err(ar.ar_reshard_plan, ok, m2n.Layout((4, 8), (3, 2), (-1, 0)), 4, domains=2) == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_reshard_plan, ok, ok, 4, domains=0) == "AR_ERR_INVALID_ARG"


def test_reshard_validates_buffers_before_launch():
    src = m2n.Layout((4, 8), (2,), (0,))
    dst = m2n.Layout((4, 8), (2, 2), (-1, 1))
    A = 1 << 40                                     # fake device addresses: every call here fails validation
    sb = [A, A + 4096]
    db = [A + 8192 * (i + 1) for i in range(4)]
    assert _err(ar.ar_reshard, [None, sb[1]], db, src, dst, 4) == "AR_ERR_INVALID_ARG"         # owner missing
    assert _err(ar.ar_reshard, sb, db[:3] + [None], src, dst, 4) == "AR_ERR_INVALID_ARG"        # destination missing
    assert _err(ar.ar_reshard, sb, [db[0] + 2] + db[1:], src, dst, 4) == "AR_ERR_ALIGNMENT"
    assert _err(ar.ar_reshard, sb, [db[0], db[0] + 32] + db[2:], src, dst, 4) == "AR_ERR_INVALID_ARG"  # dst overlap
    assert _err(ar.ar_reshard, sb, [sb[0] + 16] + db[1:], src, dst, 4) == "AR_ERR_INVALID_ARG"  # dst over a source
    with pytest.raises(ValueError):
        ar.ar_reshard(sb, db, src, dst, 4, route="nope")
    # a slot whose shard is empty (S_d < D_k) may pass NULL; the call then
    # still fails here only at the planted overlap
    tiny_src = m2n.Layout((1, 8), (2,), (0,))                   # slot 0 holds [0, 0): empty
    assert _err(ar.ar_reshard, [None, A], [A + 16], tiny_src, m2n.Layout((1, 8), (1,), (-1,)), 4) == \
        "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_reshard, [None, None], [A + 4096], tiny_src, m2n.Layout((1, 8), (1,), (-1,)), 4) == \
        "AR_ERR_INVALID_ARG"
    # a tensor with no elements is a no-op (no launch)
    empty = m2n.Layout((0, 8), (2,), (0,))
    assert _err(ar.ar_reshard, sb, db[:2], empty, m2n.Layout((0, 8), (2,), (1,)), 4) == "AR_OK"


def test_non_owner_replicas_are_never_read():
    src = m2n.Layout((4, 8), (2, 2), (-1, 0))       # slots 2, 3 replicate slots 0, 1
    p = ar.ar_reshard_plan(src, m2n.Layout((4, 8), (1,), (-1,)), 4)
    assert {s for s, *_ in p.transfers} == {0, 1}
    # a NULL entry for a replica passes validation (the call then fails only at
    # the overlap check planted here, before any launch)
    A = 1 << 40
    assert _err(ar.ar_reshard, [A, A + 4096, None, None], [A + 16], src, m2n.Layout((4, 8), (1,), (-1,)), 4) == \
        "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_reshard, [A, None, None, None], [A + 65536], src, m2n.Layout((4, 8), (1,), (-1,)), 4) == \
        "AR_ERR_INVALID_ARG"
