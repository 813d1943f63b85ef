"""The collectives under HIP graph capture: every call only enqueues kernels
on the caller's stream (no allocation, no synchronisation, no host-device
copy, no memset), so a sequence of calls can be captured once and replayed.
Each test captures through torch's graph API (torch only provides the
capture stream and the graph object), replays several times with the
inputs changed and eager work in between, and checks every replay against
the eager result of the same calls, bit for bit."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
ar = pytest.importorskip("reduce_scatter_amd")


def _capture(fn):
    """Warm up on a side stream, then capture ``fn`` into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _bits(t):
    return t.detach().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy().tobytes()


def _replays(g, inputs, outputs, eager, reps=4):
    """Replay ``g`` ``reps`` times; before each, refill ``inputs`` with fresh
    values (eager work between replays) and compute the expected outputs by
    running ``eager`` on copies; compare every output after each replay."""
    gen = torch.Generator(device="cuda")
    for rep in range(reps):
        gen.manual_seed(100 + rep)
        for x in inputs:
            if x.dtype.is_floating_point:
                x.copy_(torch.randn(x.shape, generator=gen, device="cuda").to(x.dtype))
            else:
                x.copy_(torch.randint(-1000, 1000, x.shape, generator=gen, device="cuda", dtype=x.dtype))
        torch.cuda.synchronize()
        want = eager()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outputs, want)):
            assert _bits(o) == _bits(w), "replay %d output %d differs from the eager call" % (rep, i)


@pytest.mark.parametrize("sched", ["fused", "ring", "tree", "split", "dtree", "auto"])
def test_allreduce_captured(sched):
    n, count = 8, 8 * 512 * 4 + 12
    xs = [torch.empty(count, device="cuda") for _ in range(n)]
    ys = [torch.empty(count, device="cuda") for _ in range(n)]
    X, Y = ar.pointers(xs), ar.pointers(ys)
    g = _capture(lambda: ar.ar_allreduce(X, Y, count, "f32", "sum", sched=sched))

    def eager():
        zs = [torch.empty_like(y) for y in ys]
        ar.ar_allreduce([x.clone() for x in xs], zs, count, "f32", "sum", sched=sched)
        return zs
    _replays(g, xs, ys, eager)


@pytest.mark.parametrize("sched", ["tree", "dtree"])
def test_tree_walk_captured(sched):
    """The streaming tree walk past 16 ranks (33 ranks, 2.5 MB per rank, so
    each half of the double tree is over the walk's size threshold; the
    shifted second tree walked from rank 1), captured and replayed."""
    n, count = 33, (5 << 19) // 4 + 7
    xs = [torch.empty(count, device="cuda") for _ in range(n)]
    ys = [torch.empty(count, device="cuda") for _ in range(n)]
    X, Y = ar.pointers(xs), ar.pointers(ys)
    g = _capture(lambda: ar.ar_allreduce(X, Y, count, "f32", "avg", sched=sched))

    def eager():
        zs = [torch.empty_like(y) for y in ys]
        ar.ar_allreduce([x.clone() for x in xs], zs, count, "f32", "avg", sched=sched)
        return zs
    _replays(g, xs, ys, eager)


def test_many_rank_fused_halves_captured():
    """The fused all-reduce past 16 ranks (reduce-scatter half then all-gather
    half: two launches, a ragged count) and the aligned reduce-scatter through
    the phased layout at 24 ranks (bf16), captured and replayed."""
    n, count = 40, (3 << 20) // 4 + 5
    xs = [torch.empty(count, device="cuda") for _ in range(n)]
    ys = [torch.empty(count, device="cuda") for _ in range(n)]
    X, Y = ar.pointers(xs), ar.pointers(ys)
    g = _capture(lambda: ar.ar_allreduce(X, Y, count, "f32", "avg", sched="fused"))

    def eager():
        zs = [torch.empty_like(y) for y in ys]
        ar.ar_allreduce([x.clone() for x in xs], zs, count, "f32", "avg", sched="fused")
        return zs
    _replays(g, xs, ys, eager)

    n, R = 24, 8192 + 8
    xs = [torch.empty(n * R, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    ys = [torch.empty(R, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    X, Y = ar.pointers(xs), ar.pointers(ys)
    g = _capture(lambda: ar.ar_reduce_scatter(X, Y, R, "bf16", "sum", sched="fused"))

    def eager_rs():
        zs = [torch.empty_like(y) for y in ys]
        ar.ar_reduce_scatter([x.clone() for x in xs], zs, R, "bf16", "sum", sched="fused")
        return zs
    _replays(g, xs, ys, eager_rs)


def test_reduce_scatter_then_all_gather_captured():
    n, R = 8, 4096 + 64
    xs = [torch.empty(n * R, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    ys = [torch.empty(R, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    zs = [torch.empty(n * R, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    X, Y, Z = ar.pointers(xs), ar.pointers(ys), ar.pointers(zs)

    def body():
        ar.ar_reduce_scatter(X, Y, R, "bf16", "avg")
        ar.ar_all_gather(Y, Z, R, "bf16")
    g = _capture(body)

    def eager():
        y2 = [torch.empty_like(y) for y in ys]
        z2 = [torch.empty_like(z) for z in zs]
        ar.ar_reduce_scatter([x.clone() for x in xs], y2, R, "bf16", "avg")
        ar.ar_all_gather(y2, z2, R, "bf16")
        return y2 + z2
    _replays(g, xs, ys + zs, eager)


def test_paths_off_16_byte_alignment_captured():
    """The shifted-frame all-reduce (views one element past a 16-byte
    boundary, in place) and the phased reduce-scatter / all-gather (inputs and
    outputs at their own phases, slices of a ragged length) under capture:
    vector and element-wise kernels in one graph, every replay bit for bit
    against the eager calls."""
    n, count, R = 8, 64 * 4 * 9 + 5, 64 * 8 * 3 + 3
    flat = [torch.empty(count + 1, device="cuda") for _ in range(n)]
    views = [f[1:] for f in flat]
    big = [torch.empty(n * R + 3, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    xs = [b[3:] for b in big]
    ys_t = [torch.empty(R + 1, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    ys = [y[1:] for y in ys_t]
    zs_t = [torch.empty(n * R + 5, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    zs = [z[5:] for z in zs_t]
    V, X, Y, Z = ar.pointers(views), ar.pointers(xs), ar.pointers(ys), ar.pointers(zs)

    def body():
        ar.ar_allreduce(V, V, count, "f32", "avg", sched="fused")
        ar.ar_reduce_scatter(X, Y, R, "bf16", "sum")
        ar.ar_all_gather(Y, Z, R, "bf16")
    g = _capture(body)

    def eager():
        v2 = [v.clone() for v in views]
        y2 = [torch.empty_like(y) for y in ys]
        z2 = [torch.empty_like(z) for z in zs]
        ar.ar_allreduce(v2, v2, count, "f32", "avg", sched="fused")
        ar.ar_reduce_scatter([x.clone() for x in xs], y2, R, "bf16", "sum")
        ar.ar_all_gather(y2, z2, R, "bf16")
        return v2 + y2 + z2
    _replays(g, views + xs, views + ys + zs, eager)


def test_bucket_sequence_captured():
    """Several in-place fp32 avg all-reduce calls over buckets of one flat
    buffer per rank (72 ranks), one graph for the whole sequence."""
    n = 72
    sizes = [4096, 12288 + 4, 1000, 65536]
    offs = np.concatenate([[0], np.cumsum(sizes)])
    flat = [torch.empty(int(offs[-1]), device="cuda") for _ in range(n)]
    views = [ar.pointers([f[int(offs[i]):int(offs[i + 1])] for f in flat]) for i in range(len(sizes))]
    g = _capture(lambda: [ar.ar_allreduce(v, v, c, "f32", "avg") for v, c in zip(views, sizes)])

    def eager():
        out = [f.clone() for f in flat]
        for i, c in enumerate(sizes):
            v = [o[int(offs[i]):int(offs[i + 1])] for o in out]
            ar.ar_allreduce(v, v, c, "f32", "avg")
        return out
    _replays(g, flat, flat, eager)


def test_reshard_captured():
    S = (16, 24, 40)
    src = ar.Layout(S, (2, 4), (ar.REPLICATE, 0))
    dst = ar.Layout(S, (3, 2), (ar.REPLICATE, 2), 8)
    xs = [torch.empty(ar.local_shape(src, s), device="cuda") for s in range(8)]
    ys = [torch.empty(ar.local_shape(dst, t), device="cuda") for t in range(6)]
    X, Y = ar.pointers(xs), ar.pointers(ys)
    for route in ("flat", "hier", "fused"):
        g = _capture(lambda: ar.ar_reshard(X, Y, src, dst, 4, route=route))

        def eager():
            zs = [torch.empty_like(y) for y in ys]
            ar.ar_reshard([x.clone() for x in xs], zs, src, dst, 4, route=route)
            return zs
        _replays(g, xs, ys, eager)             # the source replicas (mesh row 1) are never read


def test_default_stream_is_torchs_current_stream():
    from reduce_scatter_amd import _binding
    assert _binding._stream(None) == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert _binding._stream(None) == s.cuda_stream
    assert _binding._stream(None) == torch.cuda.current_stream().cuda_stream
