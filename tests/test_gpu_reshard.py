"""Parity of the M-to-N reshard (through the C ABI) with the oracle's
definition, byte for byte: the printed examples, random layouts of 1-3
dimensions on 1-2 axis meshes with uneven shards, every element size and
route, vector and element-wise paths, replicated sources (NULL or stale
non-owner replicas are never read), and the MoE layer workload of the NCCL
M2N paper at full size on sampled rows."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

from oracle import reshard as m2n

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
ar = pytest.importorskip("reduce_scatter_amd")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "m2n_examples.json")
ROUTES = ("flat", "hier", "fused", "auto")
NP_OF = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


def golden(name):
    with open(GOLDEN) as f:
        return json.load(f)[name]


def layout(g, side):
    d = g[side]
    return m2n.Layout(tuple(g["shape"]), tuple(d["mesh"]), tuple(d["placements"]), d["base_rank"])


def to_dev(a: np.ndarray, offset_bytes=0):
    """A device copy of ``a``'s bytes, starting ``offset_bytes`` past a
    256-byte boundary (a view into a slightly larger allocation)."""
    raw = torch.zeros(a.nbytes + offset_bytes + 16, dtype=torch.uint8, device="cuda")
    v = raw[offset_bytes:offset_bytes + a.nbytes]
    v.copy_(torch.from_numpy(np.frombuffer(np.ascontiguousarray(a).tobytes(), dtype=np.uint8).copy()))
    return v


def from_dev(t) -> bytes:
    return t.cpu().numpy().tobytes()


def random_full(rng, shape, e):
    if e == 16:
        return rng.integers(0, 2 ** 63, size=tuple(shape) + (2,), dtype=np.uint64)
    return rng.integers(0, np.iinfo(NP_OF[e]).max, size=shape, dtype=NP_OF[e], endpoint=True)


def shards_of(L, full):
    return [np.ascontiguousarray(full[m2n._box(m2n.shard_bounds(L, s))]) for s in range(L.size)]


def check(src, dst, e, rng, route, offset=0, stale_replicas=False):
    full = random_full(rng, src.shape, e)
    src_np = shards_of(src, full)
    want = shards_of(dst, full)
    owners = set(m2n.owners(src))
    src_d = []
    for s, a in enumerate(src_np):
        if s not in owners and stale_replicas:
            a = np.full_like(a, 0x5A if e == 1 else 7)            # a replica holding other data: never read
        src_d.append(to_dev(a, offset))
    dst_d = [to_dev(np.zeros_like(w), offset) for w in want]
    ar.ar_reshard(src_d, dst_d, src, dst, e, route=route)
    torch.cuda.synchronize()
    for t, w in enumerate(want):
        assert from_dev(dst_d[t]) == np.ascontiguousarray(w).tobytes(), \
            "reshard %s -> %s e=%d %s offset %d: destination slot %d differs" % (src, dst, e, route, offset, t)


def random_layout(rng, shape):
    nd_mesh = int(rng.integers(1, 3))
    mesh = tuple(int(rng.integers(1, 5)) for _ in range(nd_mesh))
    free = list(range(len(shape)))
    placements = []
    for _ in range(nd_mesh):
        if free and rng.random() < 0.7:
            placements.append(free.pop(int(rng.integers(0, len(free)))))
        else:
            placements.append(m2n.REPLICATE)
    return m2n.Layout(tuple(shape), mesh, tuple(placements), int(rng.integers(0, 9)))


def test_printed_examples_every_route():
    rng = np.random.default_rng(0)
    for name in ("example_a", "example_b", "figure3"):
        g = golden(name)
        for route in ROUTES:
            print("reshard", name, route, flush=True)
            check(layout(g, "src"), layout(g, "dst"), 4, rng, route)


@pytest.mark.parametrize("e", [1, 2, 4, 8, 16])
def test_random_layouts_every_route(e):
    rng = np.random.default_rng(100 + e)
    for it in range(60):
        nd = int(rng.integers(1, 4))
        shape = [int(rng.integers(1, 13)) for _ in range(nd)]
        if it % 2:
            shape[-1] *= 16                                     # rows of whole 16-byte vectors: the vector path
        src, dst = random_layout(rng, shape), random_layout(rng, shape)
        for route in ROUTES:
            print("reshard random", e, it, src, dst, route, flush=True)
            check(src, dst, e, rng, route)


def test_unaligned_buffers_take_the_element_path():
    rng = np.random.default_rng(7)
    src = m2n.Layout((12, 64), (4,), (0,))
    dst = m2n.Layout((12, 64), (2, 2), (-1, 1))
    for off in (2, 4, 8):
        for route in ROUTES:
            print("reshard offset", off, route, flush=True)
            check(src, dst, 2, rng, route, offset=off)


def test_non_owner_replicas_are_never_read():
    rng = np.random.default_rng(8)
    src = m2n.Layout((8, 48), (3, 4), (-1, 0))                  # 3 replicas of 4 shards
    dst = m2n.Layout((8, 48), (2, 3), (-1, 1))
    for route in ROUTES:
        check(src, dst, 4, rng, route, stale_replicas=True)
    # NULL for the replicas that are not owners
    full = random_full(rng, src.shape, 4)
    sb = [to_dev(a) if s in m2n.owners(src) else None for s, a in enumerate(shards_of(src, full))]
    want = shards_of(dst, full)
    db = [to_dev(np.zeros_like(w)) for w in want]
    ar.ar_reshard(sb, db, src, dst, 4)
    torch.cuda.synchronize()
    for t, w in enumerate(want):
        assert from_dev(db[t]) == w.tobytes()


def test_many_segments_per_shard():
    """More transfers per destination shard than one launch carries."""
    rng = np.random.default_rng(9)
    src = m2n.Layout((64, 6, 32), (2, 32), (-1, 0))
    dst = m2n.Layout((64, 6, 32), (4, 8), (-1, 2), 64)
    for route in ROUTES:
        print("reshard many", route, flush=True)
        check(src, dst, 2, rng, route)
    src = m2n.Layout((96, 8, 64), (48,), (0,))
    dst = m2n.Layout((96, 8, 64), (2, 3), (2, 1))
    for route in ROUTES:
        check(src, dst, 4, rng, route)


@pytest.mark.parametrize("rd", [2, 8])
def test_moe_layer_full_size(rd):
    """[256, 2048, 7168] bf16 (7168 MB), 16 EP sources -> TP8 x DP rd, the
    expert-sharded to tensor-parallel transfer of the paper's microbenchmark
    (TP read as sharding dimension 1).  Every destination is pre-filled with
    NaN and the sources hold values in [-1, 1), so a NaN left anywhere is an
    element not written; sampled rows are compared with their sources."""
    g = golden("moe_layer")
    S = tuple(g["shape"])
    src = m2n.Layout(S, (1, g["active_sources"]), (-1, 0))
    dst = m2n.Layout(S, (rd, g["K"]), (-1, 1), src.size)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    src_d = [(torch.rand(m2n.local_shape(src, s), generator=gen, device="cuda") * 2 - 1).to(torch.bfloat16)
             for s in range(src.size)]
    dst_d = [torch.full(m2n.local_shape(dst, t), float("nan"), dtype=torch.bfloat16, device="cuda")
             for t in range(dst.size)]
    routes = ("fused", "hier", "flat") if rd == 2 else ("fused",)
    rng = np.random.default_rng(rd)
    for route in routes:
        print("reshard moe rd=%d %s" % (rd, route), flush=True)
        for t in dst_d:
            t.fill_(float("nan"))
        ar.ar_reshard(src_d, dst_d, src, dst, 2, route=route)
        torch.cuda.synchronize()
        for t in range(dst.size):
            assert not torch.isnan(dst_d[t]).any().item(), "destination %d not fully written (%s)" % (t, route)
            b = m2n.shard_bounds(dst, t)
            for _ in range(4):
                expert = int(rng.integers(0, S[0]))
                row = int(rng.integers(0, b[1][1] - b[1][0]))
                s = expert // (S[0] // g["active_sources"])
                ls = m2n.shard_bounds(src, s)
                got = dst_d[t][expert, row].cpu()
                want = src_d[s][expert - ls[0][0], b[1][0] + row].cpu()
                assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (route, t, expert, row)
    del src_d, dst_d
    torch.cuda.empty_cache()
