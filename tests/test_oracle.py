"""Pins for the CPU oracle (``oracle/``), CPU only.

Each test ties the oracle to something other than itself: values the pages
print (``tests/golden/``), exact brute force with Python integers and
``fractions.Fraction`` on tiny inputs, closed forms the pages state, IEEE
rounding cases derived by hand from the stated hop order, and library
conversions (numpy, torch) for the oracle's own rounding code.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DTYPES = ["f32", "bf16", "f16", "i32"]
OPS = ["sum", "prod", "min", "max", "avg"]


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# helpers: typed arrays <-> exact Python values
# ---------------------------------------------------------------------------

def to_dtype(values, dtype):
    a = np.asarray(values, dtype=np.float64)
    if dtype == "f32":
        return a.astype(np.float32)
    if dtype == "f16":
        return a.astype(np.float16)
    if dtype == "i32":
        return a.astype(np.int32)
    f = a.astype(np.float32)
    assert np.all(f == a), "bf16 test values must be exact"
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "bf16 test values must be exact in bf16"
    return (bits >> 16).astype(np.uint16)


def as_float(arr, dtype):
    """Exact float64 view of a typed array."""
    if dtype == "bf16":
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return arr.astype(np.float64)


def wrap32(v: int) -> int:
    return ((v + (1 << 31)) % (1 << 32)) - (1 << 31)


def brute_int(values, op, n):
    """Direct reduction of exact Python integers, rank order 0..n-1, wrapped to int32."""
    if op in ("sum", "avg"):
        s = wrap32(sum(values))
        if op == "avg":
            q = abs(s) // n
            return -q if s < 0 else q          # C division: truncate toward zero
        return s
    if op == "prod":
        p = 1
        for v in values:
            p *= v
        return wrap32(p)
    return min(values) if op == "min" else max(values)


def gamma(k, u):
    return k * u / (1 - k * u)


UNIT_ROUNDOFF = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8 + 2.0 ** -24, "f16": 2.0 ** -11 + 2.0 ** -24}


# ---------------------------------------------------------------------------
# 1. worked examples printed on the pages, in every dtype
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_worked_example_allreduce_sum(dtype):
    g = golden("worked_examples.json")["allreduce_sum"]
    xs = [to_dtype(v, dtype) for v in g["inputs"]]
    for fn in (oracle.ring_allreduce, oracle.tree_allreduce):
        ys = fn(xs, dtype, "sum")
        for y, want in zip(ys, g["outputs"]):
            assert as_float(y, dtype).tolist() == want


@pytest.mark.parametrize("dtype", DTYPES)
def test_worked_example_reduce_scatter_avg(dtype):
    g = golden("worked_examples.json")["reduce_scatter_avg"]
    xs = [to_dtype(v, dtype) for v in g["inputs"]]
    ys = oracle.ring_reduce_scatter(xs, dtype, "avg")
    for y, want in zip(ys, g["outputs"]):
        assert as_float(y, dtype).tolist() == want
    # the full average is what all-reduce(avg) would leave on every rank
    full = oracle.ring_allreduce(xs, dtype, "avg")
    assert as_float(full[0], dtype).tolist() == g["never_assembled"]


@pytest.mark.parametrize("dtype", DTYPES)
def test_worked_example_all_gather(dtype):
    g = golden("worked_examples.json")["all_gather"]
    xs = [to_dtype(v, dtype) for v in g["inputs"]]
    ys = oracle.ring_all_gather(xs, dtype)
    for y, want in zip(ys, g["outputs"]):
        assert as_float(y, dtype).tolist() == want


def test_worked_example_gloo_route_matches_for_two_ranks():
    """The demo's CPU branch sums and then divides by the world size; with n = 2
    pre-scaling by 1/2 is exact, so both routes print the same numbers."""
    g = golden("worked_examples.json")["reduce_scatter_avg"]
    xs = [to_dtype(v, "f32") for v in g["inputs"]]
    summed = oracle.ring_reduce_scatter(xs, "f32", "sum")
    avg = oracle.ring_reduce_scatter(xs, "f32", "avg")
    for s, a in zip(summed, avg):
        assert np.array_equal(s / np.float32(2), a)


# ---------------------------------------------------------------------------
# 2. exact brute force on tiny inputs (all n in 1..9, many counts)
# ---------------------------------------------------------------------------

def _data(dtype, op, n, count, seed):
    """Per-rank data for which the reduction is exact in every dtype."""
    rg = np.random.default_rng([seed, n, count])
    if dtype == "i32":
        if op == "prod":
            return [rg.integers(-(1 << 16), 1 << 16, size=count).astype(np.int32) for _ in range(n)]
        return [rg.integers(-(1 << 30), 1 << 30, size=count).astype(np.int32) for _ in range(n)]
    if op == "prod":
        return [to_dtype(rg.choice([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0], size=count), dtype) for _ in range(n)]
    if op in ("min", "max"):
        return [to_dtype(rg.normal(size=count).astype(np.float32).astype(np.float64)
                         if dtype == "f32" else rg.integers(-100, 100, size=count), dtype) for _ in range(n)]
    return [to_dtype(rg.integers(-8, 9, size=count), dtype) for _ in range(n)]


def _brute_elem(vals, dtype, op, n):
    if dtype == "i32":
        return brute_int([int(v) for v in vals], op, n)
    fr = [Fraction(float(v)) for v in vals]
    if op == "sum":
        return sum(fr)
    if op == "avg":
        return sum(fr) / n
    if op == "prod":
        p = Fraction(1)
        for v in fr:
            p *= v
        return p
    return min(fr) if op == "min" else max(fr)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
def test_brute_force_allreduce(dtype, op):
    for n in range(1, 10):
        if op == "avg" and dtype != "i32" and n not in (1, 2, 4, 8):
            continue                       # inexact pre-scale: covered by the error-bound test
        for count in list(range(0, 21)) + [31, 37]:
            xs = _data(dtype, op, n, count, 7)
            ring = oracle.ring_allreduce(xs, dtype, op)
            tree = oracle.tree_allreduce(xs, dtype, op)
            pair = [oracle.pairwise_reduce(xs, dtype, op)] * n
            dtree = oracle.dtree_allreduce(xs, dtype, op)
            fx = [as_float(x, dtype) if dtype != "i32" else x.astype(np.int64) for x in xs]
            want = [_brute_elem([f[i] for f in fx], dtype, op, n) for i in range(count)]
            for r in range(n):
                for ys in (ring, tree, pair, dtree):
                    got = as_float(ys[r], dtype) if dtype != "i32" else ys[r].astype(np.int64)
                    assert [Fraction(float(v)) if dtype != "i32" else int(v) for v in got] == want, \
                        (dtype, op, n, count, r)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
def test_brute_force_reduce_scatter_and_all_gather(dtype, op):
    for n in range(1, 10):
        if op == "avg" and dtype != "i32" and n not in (1, 2, 4, 8):
            continue
        for R in range(0, 6):
            xs = _data(dtype, op, n, n * R, 11)
            ys = oracle.ring_reduce_scatter(xs, dtype, op)
            fx = [as_float(x, dtype) if dtype != "i32" else x.astype(np.int64) for x in xs]
            for r in range(n):
                want = [_brute_elem([f[r * R + i] for f in fx], dtype, op, n) for i in range(R)]
                got = as_float(ys[r], dtype) if dtype != "i32" else ys[r].astype(np.int64)
                assert [Fraction(float(v)) if dtype != "i32" else int(v) for v in got] == want
            # all-gather is pure assembly: bit copies of every piece, in rank order
            gs = oracle.ring_all_gather(ys, dtype)
            cat = np.concatenate(ys) if n else np.empty(0)
            for g in gs:
                assert g.tobytes() == cat.tobytes()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
def test_direct_reduce_brute_force(dtype, op):
    """The plain definition, for the cases where it is exact, against brute
    force and against the ring simulation (which must agree for these)."""
    if dtype != "i32" and op not in ("min", "max"):
        with pytest.raises(RuntimeError):
            oracle.direct_reduce([np.zeros(4, oracle.NP_DTYPE[dtype])], dtype, op)
        return
    for n in range(1, 10):
        for count in (0, 1, 5, 37):
            xs = _data(dtype, op, n, count, 17)
            y = oracle.direct_reduce(xs, dtype, op)
            fx = [as_float(x, dtype) if dtype != "i32" else x.astype(np.int64) for x in xs]
            want = [_brute_elem([f[i] for f in fx], dtype, op, n) for i in range(count)]
            got = as_float(y, dtype) if dtype != "i32" else y.astype(np.int64)
            assert [Fraction(float(v)) if dtype != "i32" else int(v) for v in got] == want
            assert y.tobytes() == oracle.ring_allreduce(xs, dtype, op)[0].tobytes() or count == 0 \
                or (op in ("min", "max") and dtype != "i32")          # +-0 ties may differ in sign


def test_c1_workload_is_exact():
    """C1: integers in [-8, 8] stored as fp32, n = 4: every sum is exact, so the
    ring, the tree and a direct integer sum agree bit for bit."""
    xs = workloads.c1_inputs()
    want = sum(x.astype(np.int64) for x in xs).astype(np.float32)
    for fn in (oracle.ring_allreduce, oracle.tree_allreduce):
        for y in fn(xs, "f32", "sum"):
            assert y.tobytes() == want.tobytes()


# ---------------------------------------------------------------------------
# 3. error bounds against exact sums (general data, order-dependent rounding)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("op", ["sum", "avg"])
def test_recursive_summation_bound(dtype, op):
    """|computed - exact| <= gamma_k * sum|x_i| (recursive summation; the avg
    pre-scale adds two more roundings: fp32(1/n) and the multiply)."""
    u = UNIT_ROUNDOFF[dtype]
    for n in (2, 3, 5, 7, 8, 9, 16, 72):
        count = 48
        xs = [workloads.normal(5, n, r, count, 1.0, dtype) for r in range(n)]
        fx = [as_float(x, dtype) for x in xs]
        for fn in (oracle.ring_allreduce, oracle.tree_allreduce):
            got = as_float(fn(xs, dtype, op)[0], dtype)
            for i in range(count):
                terms = [Fraction(f[i]) for f in fx]
                exact = sum(terms) / (n if op == "avg" else 1)
                k = (n - 1) if op == "sum" else (n + 1)
                bound = gamma(k, u) * float(sum(abs(t) for t in terms) / (n if op == "avg" else 1))
                # bf16/fp16: the final fp32 -> storage rounding of an exact value
                assert abs(Fraction(got[i]) - exact) <= Fraction(bound) + Fraction(abs(float(exact)) * u), \
                    (dtype, op, n, i)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("op", ["sum", "avg"])
def test_pairwise_summation_bound(dtype, op):
    """Pairwise summation over a tree of depth d = ceil(log2 n):
    |computed - exact| <= gamma_d * sum|x_i|; the avg pre-scale adds fp32(1/n),
    the multiply and the leaf's rounding to the storage type."""
    u = UNIT_ROUNDOFF[dtype]
    for n in (2, 3, 5, 7, 8, 9, 16, 72):
        count = 48
        xs = [workloads.normal(5, n, r, count, 1.0, dtype) for r in range(n)]
        fx = [as_float(x, dtype) for x in xs]
        got = as_float(oracle.pairwise_reduce(xs, dtype, op), dtype)
        d = math.ceil(math.log2(n))
        k = d if op == "sum" else d + 3
        for i in range(count):
            terms = [Fraction(f[i]) for f in fx]
            exact = sum(terms) / (n if op == "avg" else 1)
            bound = gamma(k, u) * float(sum(abs(t) for t in terms) / (n if op == "avg" else 1))
            assert abs(Fraction(got[i]) - exact) <= Fraction(bound) + Fraction(abs(float(exact)) * u), \
                (dtype, op, n, i)


def test_prod_relative_bound():
    u = 2.0 ** -24
    for n in (3, 5, 9, 17):
        xs = [workloads.uniform(6, n, r, 64, 0.5, 2.0, "f32") for r in range(n)]
        got = oracle.ring_allreduce(xs, "f32", "prod")[0]
        for i in range(64):
            exact = Fraction(1)
            for x in xs:
                exact *= Fraction(float(x[i]))
            assert abs(Fraction(float(got[i])) - exact) <= Fraction(gamma(n - 1, u)) * abs(exact)


def test_float_avg_power_of_two_is_scaled_sum():
    """For n = 2^k the pre-scale by 2^-k is exact (no underflow here), so
    avg == sum * 2^-k bit for bit, whatever the hop order."""
    for n in (2, 4, 8, 16):
        xs = [workloads.normal(8, n, r, 256, 1e-3, "f32") for r in range(n)]
        s = oracle.ring_allreduce(xs, "f32", "sum")[0]
        a = oracle.ring_allreduce(xs, "f32", "avg")[0]
        assert a.tobytes() == (s * np.float32(1.0 / n)).tobytes()


def test_float_avg_pre_scale_vs_sum_then_divide():
    """The two float-avg routes on the pages (pre-scale by 1/n as read; the
    demo's sum-then-divide) agree closely for n = 72 but not bit for bit."""
    n = 72
    xs = [workloads.normal(9, 0, r, 4096, 1e-3, "f32") for r in range(n)]
    a = oracle.ring_allreduce(xs, "f32", "avg")[0].astype(np.float64)
    s = (oracle.ring_allreduce(xs, "f32", "sum")[0] / np.float32(n)).astype(np.float64)
    scale = np.abs(s).max()
    assert np.max(np.abs(a - s)) <= 1e-5 * scale
    assert not np.array_equal(a, s)      # the reading matters: the routes differ


# Hand-derived float-avg values at rank counts that are not powers of two
# ("NCCL all-reduce", section "What all-reduce promises": a floating-point
# contribution is pre-scaled by 1/n as it is read).  With one non-zero
# contribution x and zeros elsewhere every add is exact, so the result is
# fp32(x * s) with s = fp32(1/n), computed by hand:
#   n = 3:  2^25 / 3 = 11184810.67 -> s = 11184811 * 2^-25 (0x3EAAAAAB).
#           x = 5: 5s = 55924055 * 2^-25; in [1, 2) the spacing is 2^-23 = 4 * 2^-25
#           and 55924055 / 4 = 13981013.75 -> 13981014 * 2^-23 = 0x3FD55556,
#           while x / 3 = 13981013.33 * 2^-23 -> 0x3FD55555.
#   n = 72: 2^30 / 72 = 14913080.89 -> s = 14913081 * 2^-30 (0x3C638E39).
#           x = 17: 17s = 253522377 * 2^-30; in [1/8, 1/4) the spacing is 2^-26
#           and 253522377 / 16 = 15845148.56 -> 15845149 * 2^-26 = 0x3E71C71D,
#           while 17 / 72 = 15845148.44 * 2^-26 -> 0x3E71C71C.
# A per-contribution x / n, or a sum divided by n at the end, gives the second
# pattern in both cases.
PRESCALE_CASES = [(3, 5.0, 0x3FD55556, 0x3FD55555), (72, 17.0, 0x3E71C71D, 0x3E71C71C)]


@pytest.mark.parametrize("n,x,want,divided", PRESCALE_CASES)
def test_float_avg_prescale_hand_cases(n, x, want, divided):
    assert np.float32(1.0 / n).view(np.uint32) == (0x3EAAAAAB if n == 3 else 0x3C638E39)
    count = 4 * n + 3                               # every chunk, and a ragged tail
    for holder in (0, n // 2, n - 1):
        xs = [np.zeros(count, np.float32) for _ in range(n)]
        xs[holder][:] = x
        outs = [oracle.ring_allreduce(xs, "f32", "avg")[0], oracle.tree_allreduce(xs, "f32", "avg")[0],
                oracle.dtree_allreduce(xs, "f32", "avg")[0], oracle.pairwise_reduce(xs, "f32", "avg")]
        rs = oracle.ring_reduce_scatter([np.full(n * 3, x if r == holder else 0.0, np.float32) for r in range(n)],
                                        "f32", "avg")
        for y in outs + rs:
            assert set(y.view(np.uint32).tolist()) == {want}, (n, holder, sorted(set(y.view(np.uint32).tolist())))
            assert want != divided


# ---------------------------------------------------------------------------
# 4. the hop order, pinned by IEEE rounding cases derived by hand
# ---------------------------------------------------------------------------
#
# With B = 2^p (p = 24 for fp32, 8 for bf16, 11 for fp16: the first power of
# two whose ulp is 2), B + 1 is a tie that rounds back to B (even), while
# 1 - B = -(B - 1) is exact.  Take contributions {+B, -B, +1} with zeros on
# the other ranks and add them left to right with per-hop rounding:
#   +B .. 1 .. -B  ->  (B + 1) - B = 0        1 .. +B .. -B  ->  (1 + B) - B = 0
#   +B .. -B .. 1  ->  0 + 1 = 1              -B first, or 1 .. -B .. +B  ->  1
# so the result is 0 exactly when +B and the 1 both come before -B.  The
# expected values below apply that rule to the stated order: chunk c's chain
# is ranks c+1, c+2, ..., c (mod n).

BIG = {"f32": 2.0 ** 24, "bf16": 2.0 ** 8, "f16": 2.0 ** 11}


def _chain_result(chain, pos_big, pos_neg, pos_one):
    i_b, i_n, i_1 = chain.index(pos_big), chain.index(pos_neg), chain.index(pos_one)
    return 0.0 if (i_b < i_n and i_1 < i_n) else 1.0


def _stated_chain(n, c):
    return [(c + k) % n for k in range(1, n + 1)]


def _order_cases(dtype, n, trials, seed, chain_of=_stated_chain):
    B = BIG[dtype]
    u = 16 // (4 if dtype == "f32" else 2)
    count = n * u                                      # chunk c = elements [c*u, (c+1)*u)
    rg = np.random.default_rng(seed)
    cases = []
    for _ in range(trials):
        xs = [np.zeros(count) for _ in range(n)]
        expect = np.zeros(count)
        for c in range(n):
            pb, pn, p1 = (int(v) for v in rg.choice(n, size=3, replace=False))
            for i in range(c * u, (c + 1) * u):
                xs[pb][i], xs[pn][i], xs[p1][i] = B, -B, 1.0
                expect[i] = _chain_result(chain_of(n, c), pb, pn, p1)
        cases.append((xs, expect))
    return cases


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_ring_hop_order_rounding_cases(dtype):
    for n in (3, 4, 5, 8):
        u = 16 // (4 if dtype == "f32" else 2)
        assert oracle.allreduce_chunks(dtype, n, n * u) == [c * u for c in range(n + 1)]
        for xs, expect in _order_cases(dtype, n, 12, n):
            for y in oracle.ring_allreduce([to_dtype(x, dtype) for x in xs], dtype, "sum"):
                assert as_float(y, dtype).tolist() == expect.tolist(), (dtype, n)


def test_ring_hop_order_cases_have_power():
    """The same cases, with the two nearest misreadings of the order (the chain
    starts at the owner; every chunk in rank order 0..n-1), predict different
    results, so the test above would catch either mistake."""
    owner_first = lambda n, c: [(c + k) % n for k in range(n)]
    rank_order = lambda n, c: list(range(n))
    for n in (3, 4, 5, 8):
        stated = [e for _, e in _order_cases("f32", n, 12, n)]
        for alt in (owner_first, rank_order):
            other = [e for _, e in _order_cases("f32", n, 12, n, chain_of=alt)]
            assert any(not np.array_equal(a, b) for a, b in zip(stated, other)), n


def test_bf16_rounds_at_every_hop():
    """bf16 partials are rounded to bf16 after each hop: 256 + 1 -> 256, so
    (256 + 1) - 256 = 0, where an fp32 accumulator would give 1."""
    n, u = 3, 8
    xs = [np.zeros(n * u) for _ in range(n)]
    # chunk 0's chain is 1, 2, 0
    xs[1][:u], xs[2][:u], xs[0][:u] = 256.0, 1.0, -256.0
    y = oracle.ring_allreduce([to_dtype(x, "bf16") for x in xs], "bf16", "sum")[0]
    assert as_float(y, "bf16")[:u].tolist() == [0.0] * u
    y32 = oracle.ring_allreduce([x.astype(np.float32) for x in xs], "f32", "sum")[0]
    assert y32[:u].tolist() == [1.0] * u


def test_min_max_ties_keep_incoming():
    """min/max keep the incoming partial on ties: visible with -0.0 and +0.0."""
    n, u = 2, 4
    # chunk 0's chain: rank 1 then rank 0.  incoming = rank 1's value.
    a = np.zeros(n * u, np.float32)
    b = np.zeros(n * u, np.float32)
    b[:u] = -0.0
    ymin = oracle.ring_allreduce([a, b], "f32", "min")[0]
    ymax = oracle.ring_allreduce([a, b], "f32", "max")[0]
    assert np.signbit(ymin[:u]).all() and np.signbit(ymax[:u]).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_two_ranks_is_one_ieee_operation(dtype):
    """With n = 2 every element is a single operation, so each result equals the
    library's own correctly rounded operation in that dtype (numpy for fp32
    and fp16, torch for bf16)."""
    import torch
    count = 4096
    xs = [workloads.normal(10, 0, r, count, 1.0, dtype) for r in range(2)]
    fx = [as_float(x, dtype) for x in xs]
    for op in ("sum", "prod", "avg"):
        got = as_float(oracle.ring_allreduce(xs, dtype, op)[0], dtype)
        if dtype == "bf16":
            ta = torch.tensor(fx[0], dtype=torch.float32).to(torch.bfloat16)
            tb = torch.tensor(fx[1], dtype=torch.float32).to(torch.bfloat16)
            if op == "avg":
                ta, tb = (ta.float() * 0.5).to(torch.bfloat16), (tb.float() * 0.5).to(torch.bfloat16)
            r = (ta + tb) if op != "prod" else (ta * tb)
            want = r.float().numpy().astype(np.float64)
        else:
            npd = np.float32 if dtype == "f32" else np.float16
            a, b = fx[0].astype(npd), fx[1].astype(npd)
            if op == "avg":
                a, b = a * npd(0.5), b * npd(0.5)
            want = ((a + b) if op != "prod" else (a * b)).astype(np.float64)
        # chunk 0 is summed as rank1 (+) rank0, chunk 1 as rank0 (+) rank1: the same for + and *
        assert np.array_equal(got, want), (dtype, op)


# ---------------------------------------------------------------------------
# 5. closed forms: hop counts and bytes on the wire
# ---------------------------------------------------------------------------

def test_ring_hops_and_bytes_closed_forms():
    cf = golden("closed_forms.json")["ring_steps"]["n_to_hops"]
    for n in (2, 3, 4, 8, 16):
        count = n * 4 * 3
        xs = [np.ones(count, np.float32) for _ in range(n)]
        _, hops, sent = oracle.ring_allreduce(xs, "f32", "sum", counters=True)
        assert hops == [2 * (n - 1)] * n
        S = count * 4
        assert sent == [2 * (n - 1) * S // n] * n          # a hair under 2S per rank
        if str(n) in cf:
            assert hops[0] == cf[str(n)]
    assert 2 * (1024 - 1) == cf["1024"]
    # reduce-scatter and all-gather each move half of that
    n, R = 8, 12
    xs = [np.ones(n * R, np.float32) for _ in range(n)]
    ys, hops, sent = oracle.ring_reduce_scatter(xs, "f32", "sum", counters=True)
    assert hops == [n - 1] * n and sent == [(n - 1) * R * 4] * n
    _, hops, sent = oracle.ring_all_gather(ys, "f32", counters=True)
    assert hops == [n - 1] * n and sent == [(n - 1) * R * 4] * n


def test_allreduce_chunks_16_byte_units():
    for dtype, u in (("f32", 4), ("bf16", 8), ("i32", 4)):
        for n in (1, 3, 8, 72):
            for count in (0, 1, 5, 17, 1000, 4099, 25 * 2 ** 20 // 4):
                off = oracle.allreduce_chunks(dtype, n, count)
                assert off[0] == 0 and off[-1] == count and len(off) == n + 1
                assert all(a <= b for a, b in zip(off, off[1:]))
                assert all(o % u == 0 for o in off[:-1])
                V = -(-count // u)
                lens = [-(-min(count, b) // u) * u - a for a, b in zip(off, off[1:])]
                assert max(lens) - min(lens) <= u if V >= n else True
                if count % (n * u) == 0:
                    assert off == [c * count // n for c in range(n + 1)]


def test_allreduce_chunks_floor_cut_hand_cases():
    """Chunk bounds at counts that n*u does not divide, evaluated by hand from
    the floor of Eq. (2) (M2N paper, section IV 'Local shard bounds') in 16-byte
    units (tests/golden/chunk_bounds.json); a ceiling cut fails every case but
    the exact one."""
    g = golden("chunk_bounds.json")
    for case in g["cases"]:
        got = oracle.allreduce_chunks(case["dtype"], case["n"], case["count"])
        assert got == case["bounds"], case
        if case["ceil"] != case["bounds"]:
            assert got != case["ceil"]
    b = g["c5_bucket"]
    got = oracle.allreduce_chunks(b["dtype"], b["n"], b["count"])
    for c, v in b["bounds_at"].items():
        assert got[int(c)] == v, (c, got[int(c)], v)
    for c, v in b["ceil_at"].items():
        assert got[int(c)] != v
    lens = [(got[c + 1] - got[c]) // 4 for c in range(b["n"])]
    assert [c for c in range(b["n"]) if lens[c] == 21716] == b["long_chunks"]
    assert all(v in (21715, 21716) for v in lens)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_floor_cut_decides_the_hop_order_of_the_cut_vectors(dtype):
    """The cut changes results, not only bounds.  n = 3, 5 vectors per rank:
    the floor cut gives chunks of 1, 2 and 2 vectors, a ceiling cut 2, 2 and 1.
    Vector 1 is in chunk 1 (chain 2, 0, 1) under the floor and in chunk 0
    (chain 1, 2, 0) under the ceiling; vector 3 is in chunk 2 (chain 0, 1, 2)
    under the floor and in chunk 1 under the ceiling.  The +B / 1 / -B rule of
    the hop-order cases (the result is 0 exactly when +B and the 1 both come
    before -B) then gives 0 for the stated cut and 1 for the other."""
    n = 3
    u = 16 // (4 if dtype == "f32" else 2)
    B = BIG[dtype]
    count = 5 * u
    xs = [np.zeros(count) for _ in range(n)]
    v1 = slice(1 * u, 2 * u)          # floor: chunk 1 = ranks 2, 0, 1
    xs[2][v1], xs[0][v1], xs[1][v1] = B, 1.0, -B
    v3 = slice(3 * u, 4 * u)          # floor: chunk 2 = ranks 0, 1, 2
    xs[0][v3], xs[1][v3], xs[2][v3] = B, 1.0, -B
    assert oracle.allreduce_chunks(dtype, n, count) == [0, u, 3 * u, 5 * u]
    for y in oracle.ring_allreduce([to_dtype(x, dtype) for x in xs], dtype, "sum"):
        assert as_float(y, dtype).tolist() == [0.0] * count, dtype
    # with the owner's rank in the ceiling cut's chains the same vectors give 1
    ceil_chain = {1: [1, 2, 0], 3: [2, 0, 1]}
    assert _chain_result(ceil_chain[1], 2, 1, 0) == 1.0 and _chain_result(ceil_chain[3], 0, 2, 1) == 1.0


# ---------------------------------------------------------------------------
# 6. the tree
# ---------------------------------------------------------------------------

def test_tree_matches_the_14_rank_picture():
    g = golden("tree14.json")
    n = g["n"]
    parent = [oracle.tree_parent(n, v) for v in range(n)]
    assert parent == g["parent"]
    children = {v: [c for c in range(n) if parent[c] == v] for v in range(n)}
    assert sorted(v for v in range(n) if not children[v]) == g["leaves"]


def _depth(n):
    d = 0
    for v in range(n):
        k, p = 0, v
        while p != 0:
            p = oracle.tree_parent(n, p)
            k += 1
            assert k <= n
        d = max(d, k)
    return d


def test_tree_shape_for_all_small_n():
    cf = golden("closed_forms.json")["tree_depth"]["n_to_depth"]
    for n in range(1, 130):
        parent = [oracle.tree_parent(n, v) for v in range(n)]
        assert parent[0] == -1
        assert all(0 <= parent[v] < n for v in range(1, n))
        nchild = [sum(1 for c in range(n) if parent[c] == v) for v in range(n)]
        assert max(nchild) <= 2
        assert _depth(n) == (math.ceil(math.log2(n)) if n > 1 else 0)
    assert _depth(1024) == cf["1024"]


def test_tree_order_own_first_then_children_ascending():
    """n = 4: parent(1) = parent(3) = 2, parent(2) = 0, so the root value is
    x0 + ((x2 + x1) + x3).  Cases derived by hand with B = 2^24:
      x2 = B, x1 = 1, x3 = -B: (B + 1) -> B, B - B = 0            -> 0
        (children first, (x1 + x3) + x2 = (1 - B) + B, would give 1;
         children descending, (x2 + x3) + x1 = 0 + 1, would give 1)
      x2 = 1, x1 = -B, x3 = B: (1 - B) exact, + B = 1             -> 1
      x0 = -B, x2 = B, x1 = x3 = 0: 0 + 0, then -B + B = 0        -> 0
      x0 = 1, x1 = B, x3 = -B, x2 = 0: (0 + B) - B = 0, 1 + 0     -> 1"""
    B = 2.0 ** 24

    def run(x0, x1, x2, x3):
        xs = [np.full(4, v, np.float32) for v in (x0, x1, x2, x3)]
        out = oracle.tree_allreduce(xs, "f32", "sum")
        assert all(o.tobytes() == out[0].tobytes() for o in out)
        return float(out[3][0])

    assert [oracle.tree_parent(4, v) for v in range(4)] == [-1, 2, 0, 2]
    assert run(0.0, 1.0, B, -B) == 0.0
    assert run(0.0, -B, 1.0, B) == 1.0
    assert run(-B, 0.0, B, 0.0) == 0.0
    assert run(1.0, B, 0.0, -B) == 1.0


def test_tree_and_ring_agree_when_exact_and_within_bound_otherwise():
    n = 8
    xs = [workloads.normal(12, 0, r, 1024, 1e-3, "f32") for r in range(n)]
    ring = oracle.ring_allreduce(xs, "f32", "sum")[0].astype(np.float64)
    tree = oracle.tree_allreduce(xs, "f32", "sum")[0].astype(np.float64)
    assert np.max(np.abs(ring - tree)) <= 1e-6 * np.max(np.abs(ring))


# ---------------------------------------------------------------------------
# 6a. the double binary tree
# ---------------------------------------------------------------------------

def _bit_trick_parent(n, v):
    """The first tree as the pages describe it (lowest set bit fixes the depth;
    clear it and set the next bit up, or just clear it past the end)."""
    if v == 0:
        return -1
    b = v & -v
    p = (v ^ b) | (b << 1)
    return v ^ b if p >= n else p


def _second_tree_parent(n, v):
    """The mirror image of the first tree for even n, the first tree shifted by
    one rank (+1) for odd n."""
    if n % 2 == 0:
        p = _bit_trick_parent(n, n - 1 - v)
        return -1 if p < 0 else n - 1 - p
    p = _bit_trick_parent(n, (v - 1) % n)
    return -1 if p < 0 else (p + 1) % n


def test_dtree_parents_follow_the_construction():
    for n in range(1, 129):
        for which, ref in ((0, _bit_trick_parent), (1, _second_tree_parent)):
            assert [oracle.dtree_parent(n, which, v) for v in range(n)] == [ref(n, v) for v in range(n)], (n, which)


def test_dtree_second_tree_mirrors_the_14_rank_picture():
    g = golden("tree14.json")
    n, par = g["n"], g["parent"]
    want = [-1 if par[n - 1 - v] < 0 else n - 1 - par[n - 1 - v] for v in range(n)]
    assert [oracle.dtree_parent(n, 1, v) for v in range(n)] == want


def test_dtree_trees_are_complementary():
    """Every rank is interior in at most one of the two trees, except one
    boundary rank interior in both when n is odd; both trees are ceil(log2 n)
    deep, with at most two children per node; the first tree's leaves are the
    odd ranks."""
    for n in range(2, 129):
        interior = []
        for which in (0, 1):
            par = [oracle.dtree_parent(n, which, v) for v in range(n)]
            assert sum(p < 0 for p in par) == 1
            kids = {v: [c for c in range(n) if par[c] == v] for v in range(n)}
            assert max(len(k) for k in kids.values()) <= 2
            depth = 0
            for v in range(n):
                d, u = 0, v
                while par[u] >= 0:
                    u, d = par[u], d + 1
                    assert d <= n
                depth = max(depth, d)
            assert depth == math.ceil(math.log2(n)), (n, which)
            interior.append({v for v in range(n) if kids[v]})
        both = interior[0] & interior[1]
        assert len(both) == (n % 2), (n, both)
        assert {v for v in range(n) if v not in interior[0]} == {v for v in range(1, n, 2)}


def _first_pair(par, a, b, c):
    """Of three ranks holding the only non-zero contributions, the two whose
    values are combined first in a tree reduce (own value first, then children
    in ascending rank order): the pair with the deepest lowest common ancestor;
    when all three share it, the ancestor's own value and the one in its
    lower-ranked child's subtree."""
    def chain(v):
        out = [v]
        while par[out[-1]] >= 0:
            out.append(par[out[-1]])
        return out

    def lca(x, y):
        cx = chain(x)
        return next(v for v in chain(y) if v in cx)
    pairs = [(a, b), (a, c), (b, c)]
    depth = {p: len(chain(lca(*p))) for p in pairs}
    deepest = max(depth.values())
    best = [p for p in pairs if depth[p] == deepest]
    if len(best) == 1:
        return set(best[0])
    m = lca(a, b)                                      # all three meet at m, in three slots
    kids = sorted(v for v in range(len(par)) if par[v] == m)
    slot = {}
    for x in (a, b, c):
        slot[x] = 0 if x == m else 1 + next(i for i, k in enumerate(kids) if m != x and k in chain(x))
    order = sorted((a, b, c), key=slot.get)
    return {order[0], order[1]}


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_dtree_rounding_cases_on_both_halves(dtype):
    """+B, -B, +1 on three ranks (zeros elsewhere): the result is 0 exactly when
    +B and 1 are combined first.  Elements [0, u*floor(V/2)) follow the first
    tree, the rest the second, including a ragged count."""
    B = BIG[dtype]
    u = 16 // (4 if dtype == "f32" else 2)
    for n in (3, 5, 6, 8, 13, 14):
        trees = [[_bit_trick_parent(n, v) for v in range(n)], [_second_tree_parent(n, v) for v in range(n)]]
        for count in (u * 12, u * 13, u * 13 + 3):
            rg = np.random.default_rng([n, count])
            xs = [np.zeros(count) for _ in range(n)]
            expect = np.zeros(count)
            V = -(-count // u)
            half = u * (V // 2)
            place = []
            for i in range(count):
                pb, pn, p1 = (int(v) for v in rg.choice(n, size=3, replace=False))
                xs[pb][i], xs[pn][i], xs[p1][i] = B, -B, 1.0
                place.append((pb, pn, p1))
                expect[i] = 0.0 if _first_pair(trees[0 if i < half else 1], pb, pn, p1) == {pb, p1} else 1.0
            got = oracle.dtree_allreduce([to_dtype(x, dtype) for x in xs], dtype, "sum")
            for y in got:
                assert as_float(y, dtype).tolist() == expect.tolist(), (dtype, n, count)
            # the cases tell the trees apart: the other tree predicts otherwise somewhere in each half
            other = [0.0 if _first_pair(trees[1 if i < half else 0], pb, pn, p1) == {pb, p1} else 1.0
                     for i, (pb, pn, p1) in enumerate(place)]
            if n > 3:
                assert other[:half] != expect[:half].tolist() and other[half:] != expect[half:].tolist(), (n, count)


def test_dtree_first_half_is_the_single_tree():
    for n in (2, 5, 8, 16, 72):
        count = 4 * 40 + 3
        xs = [workloads.normal(12, n, r, count, 1.0, "f32") for r in range(n)]
        d = oracle.dtree_allreduce(xs, "f32", "sum")[0]
        t = oracle.tree_allreduce(xs, "f32", "sum")[0]
        half = 4 * ((-(-count // 4)) // 2)
        assert d[:half].tobytes() == t[:half].tobytes()
        if n > 2:
            assert d[half:].tobytes() != t[half:].tobytes()


# ---------------------------------------------------------------------------
# 6b. the all-ranks-at-once fused pass: the aligned pairwise order
# ---------------------------------------------------------------------------
#
# In the aligned binary tree over rank indices, leaves i and j first meet at
# the level given by the highest bit in which i and j differ, i.e.
# (i ^ j).bit_length(); of three leaves, exactly one pair meets strictly
# first.  With contributions {+B, -B, +1} and zeros elsewhere (B as in
# section 4), adding zero is exact, so the result is (B + 1) - B = 0 when +B
# and the 1 meet first, and 1 when either other pair meets first.  This
# closed form is independent of the oracle's recursion.

def _meet(i, j):
    return (i ^ j).bit_length()


def _pairwise_rule(pb, pn, p1):
    return 0.0 if _meet(pb, p1) < min(_meet(pb, pn), _meet(p1, pn)) else 1.0


def _pairwise_cases(dtype, n, trials, seed):
    B = BIG[dtype]
    rg = np.random.default_rng(seed)
    xs = [np.zeros(trials) for _ in range(n)]
    expect = np.zeros(trials)
    placements = []
    for i in range(trials):
        pb, pn, p1 = (int(v) for v in rg.choice(n, size=3, replace=False))
        xs[pb][i], xs[pn][i], xs[p1][i] = B, -B, 1.0
        expect[i] = _pairwise_rule(pb, pn, p1)
        placements.append((pb, pn, p1))
    return xs, expect, placements


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_pairwise_rounding_cases(dtype):
    for n in (3, 4, 5, 6, 7, 8, 13, 16, 72, 128):
        xs, expect, _ = _pairwise_cases(dtype, n, 64, n)
        got = oracle.pairwise_reduce([to_dtype(x, dtype) for x in xs], dtype, "sum")
        assert as_float(got, dtype).tolist() == expect.tolist(), (dtype, n)
        assert 0.0 in expect and 1.0 in expect


def _eval_tree(split, vals):
    """fp32 evaluation of a combine tree given by ``split(lo, len) -> h``."""
    def rec(lo, ln):
        if ln == 1:
            return np.float32(vals[lo])
        h = split(lo, ln)
        return np.float32(rec(lo, h) + rec(lo + h, ln - h))
    return float(rec(0, len(vals)))


def test_pairwise_cases_have_power():
    """The nearest misreadings (split a range in halves rather than at a power
    of two; rank order 0..n-1; the ring's order for chunk 0) predict other
    results on these cases, so the test above would catch each of them."""
    halves = lambda lo, ln: ln // 2
    chain = lambda lo, ln: ln - 1                  # ((x0 + x1) + x2) + ...
    for n in (6, 7, 13, 72):
        xs, expect, placements = _pairwise_cases("f32", n, 64, n)
        vals = [[x[i] for x in xs] for i in range(len(expect))]
        for alt in (halves, chain):
            assert any(_eval_tree(alt, v) != e for v, e in zip(vals, expect)), n
        ring_pred = [_eval_tree(chain, v[1:] + v[:1]) for v in vals]   # chunk 0: ranks 1, ..., n-1, 0
        assert any(a != b for a, b in zip(ring_pred, expect)), n


def test_pairwise_worked_cases():
    """Hand-evaluated cases: n = 3 combines (x0 + x1) + x2; n = 6 combines
    (x0..x3) with (x4, x5); n = 72 combines ranks 0..63 with 64..71."""
    t = 2.0 ** -24
    cases = [
        ([1.0, t, t], 1.0),                        # (1 + t) -> 1, 1 + t -> 1;  1 + (t + t) would be 1 + 2t
        ([1.0, 0.0, t, t], 1.0 + 2 * t),           # (1 + 0) + (t + t)
        ([1.0, 0.0, 0.0, t, t, 0.0], 1.0),         # ((1+0)+(0+t)) + (t+0): halves would give 1 + 2t
    ]
    x72 = [0.0] * 72
    x72[0], x72[63], x72[64] = 1.0, t, t           # ranks 0..63 -> 1 + t -> 1; then + t -> 1
    cases.append((x72, 1.0))
    for vals, want in cases:
        xs = [np.array([v], np.float32) for v in vals]
        assert float(oracle.pairwise_reduce(xs, "f32", "sum")[0]) == want, vals


def test_pairwise_min_max_ties_keep_lower_ranks():
    a, b = np.zeros(4, np.float32), np.full(4, -0.0, np.float32)
    assert not np.signbit(oracle.pairwise_reduce([a, b], "f32", "min")).any()
    assert np.signbit(oracle.pairwise_reduce([b, a], "f32", "min")).all()
    assert np.signbit(oracle.pairwise_reduce([b, a], "f32", "max")).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_pairwise_two_ranks_is_the_ring(dtype):
    """n = 2: one operation per element, which the ring also computes (and the
    ring's n = 2 result is pinned to the library's own operation above)."""
    xs = [workloads.normal(10, 0, r, 4096, 1.0, dtype) for r in range(2)]
    for op in ("sum", "prod", "avg"):
        want = oracle.ring_allreduce(xs, dtype, op)[0]
        assert oracle.pairwise_reduce(xs, dtype, op).tobytes() == want.tobytes(), (dtype, op)


def test_pairwise_power_of_two_avg_is_scaled_sum():
    for n in (4, 8, 16, 64):
        xs = [workloads.normal(8, n, r, 256, 1e-3, "f32") for r in range(n)]
        s = oracle.pairwise_reduce(xs, "f32", "sum")
        a = oracle.pairwise_reduce(xs, "f32", "avg")
        assert a.tobytes() == (s * np.float32(1.0 / n)).tobytes()


# ---------------------------------------------------------------------------
# 6c. numerics variants: fp32 accumulation, split avg divisor
# ---------------------------------------------------------------------------

def test_split_p_is_the_power_of_two_nearest_above_sqrt_n():
    for n in range(1, 129):
        p = oracle.split_p(n)
        assert p & (p - 1) == 0 and p * p >= n and (p == 1 or (p // 2) ** 2 < n), (n, p)
    assert [oracle.split_p(n) for n in (2, 4, 8, 16, 72)] == [2, 2, 4, 4, 16]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_acc32_keeps_what_per_hop_rounding_loses(dtype):
    """Chunk 0's chain is ranks 1, 2, 0: B + 1 - B.  Rounded to the storage
    type after each hop it is 0 (B + 1 ties back to B); with fp32 partials it is
    the exact 1."""
    B = BIG[dtype]
    n, u = 3, 8
    xs = [np.zeros(n * u) for _ in range(n)]
    xs[1][:u], xs[2][:u], xs[0][:u] = B, 1.0, -B
    t = [to_dtype(x, dtype) for x in xs]
    assert as_float(oracle.ring_allreduce(t, dtype, "sum")[0], dtype)[:u].tolist() == [0.0] * u
    for fn in (lambda: oracle.ring_allreduce(t, dtype, "sum", acc32=True)[0],
               lambda: oracle.ring_reduce_scatter(t, dtype, "sum", acc32=True)[0]):
        assert as_float(fn(), dtype)[:u].tolist() == [1.0] * u


def _round_once(values_f64, dtype):
    """Storage-type rounding by library code: numpy for fp16, torch for bf16."""
    if dtype == "f16":
        return values_f64.astype(np.float32).astype(np.float16).astype(np.float64)
    import torch
    return torch.tensor(values_f64.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("op", ["sum", "prod", "avg", "max"])
def test_acc32_is_the_fp32_ring_rounded_once(dtype, op):
    """fp32 partials in the ring's hop order, rounded once: the fp32 ring (pinned
    above) on the widened inputs, rounded by numpy / torch."""
    for n in (2, 5, 8, 16, 72):
        count = n * 8 * 3 + 5
        kind = "pos" if op == "prod" else "normal"
        xs = [workloads.random_values(13, n, r, count, dtype, kind) for r in range(n)]
        wide = [as_float(x, dtype).astype(np.float32) for x in xs]
        want = _round_once(oracle.ring_allreduce(wide, "f32", op)[0].astype(np.float64), dtype)
        got = as_float(oracle.ring_allreduce(xs, dtype, op, acc32=True)[0], dtype)
        assert got.tolist() == want.tolist(), (dtype, op, n)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_acc32_error_bound_and_the_per_hop_loss(dtype):
    """With fp32 partials the error is one storage rounding plus fp32's
    recursive-summation bound; per-hop storage rounding exceeds that bound at
    72 ranks (the loss the pages attribute to bf16 accumulation)."""
    n, count = 72, 512
    xs = [workloads.normal(14, n, r, count, 1.0, dtype) for r in range(n)]
    fx = [as_float(x, dtype) for x in xs]
    uT = UNIT_ROUNDOFF[dtype]
    acc = as_float(oracle.ring_allreduce(xs, dtype, "sum", acc32=True)[0], dtype)
    hop = as_float(oracle.ring_allreduce(xs, dtype, "sum")[0], dtype)
    worst_hop = 0.0
    for i in range(count):
        terms = [Fraction(f[i]) for f in fx]
        exact = sum(terms)
        bound = Fraction(abs(float(exact)) * uT) + Fraction(gamma(n - 1, 2.0 ** -24) * float(sum(abs(t) for t in terms)))
        assert abs(Fraction(acc[i]) - exact) <= bound * (1 + uT), i
        worst_hop = max(worst_hop, float(abs(Fraction(hop[i]) - exact) / bound))
    assert worst_hop > 1.0


def test_acc32_is_a_no_op_for_fp32_and_int32():
    for dtype in ("f32", "i32"):
        xs = [workloads.random_values(15, 6, r, 301, dtype) for r in range(6)]
        for op in OPS:
            a = oracle.ring_allreduce(xs, dtype, op)[0]
            b = oracle.ring_allreduce(xs, dtype, op, acc32=True)[0]
            assert a.tobytes() == b.tobytes(), (dtype, op)


def test_avg_split_fp16_keeps_what_the_prescale_underflows():
    """fp16, n = 8 (p = 4, q = 2), every contribution 2^-22: pre-scaled by 1/8
    each is 2^-25, half the smallest subnormal, which rounds (to even) to 0;
    split, each is 2^-24, the sum 2^-21 and the average the exact 2^-22."""
    n = 8
    xs = [np.full(64, 2.0 ** -22, np.float16) for _ in range(n)]
    for fn in (oracle.ring_allreduce, oracle.tree_allreduce, oracle.dtree_allreduce):
        assert fn(xs, "f16", "avg")[0].astype(np.float64).tolist() == [0.0] * 64
        assert fn(xs, "f16", "avg", avg_split=True)[0].astype(np.float64).tolist() == [2.0 ** -22] * 64
    assert oracle.pairwise_reduce(xs, "f16", "avg", avg_split=True).astype(np.float64).tolist() == [2.0 ** -22] * 64


def test_avg_split_fp16_overflows_where_the_prescale_does_not():
    """The other side of the trade: n = 16 (p = q = 4), every contribution 2^15:
    pre-scaled by 1/16 each is 2048 and every partial sum a multiple of 2048,
    exact in fp16, so the average is 2^15; split, each is 8192 and the partial
    sums pass the fp16 maximum 65504 (8 * 8192 = 65536 rounds to +inf)."""
    xs = [np.full(64, 32768.0, np.float16) for _ in range(16)]
    assert oracle.ring_allreduce(xs, "f16", "avg")[0].astype(np.float64).tolist() == [32768.0] * 64
    assert np.isposinf(oracle.ring_allreduce(xs, "f16", "avg", avg_split=True)[0].astype(np.float64)).all()


def test_avg_split_equals_the_prescale_when_both_factors_are_exact():
    """n = 4^k: p = q = 2^k, so x/p and sum/q are exact power-of-two scalings and
    the split route gives the pre-scale route's bits (fp32, no under/overflow)."""
    for n in (4, 16, 64):
        xs = [workloads.normal(16, n, r, 300, 1e-3, "f32") for r in range(n)]
        for fn in (lambda **k: oracle.ring_allreduce(xs, "f32", "avg", **k)[0],
                   lambda **k: oracle.tree_allreduce(xs, "f32", "avg", **k)[0],
                   lambda **k: oracle.pairwise_reduce(xs, "f32", "avg", **k)):
            assert fn().tobytes() == fn(avg_split=True).tobytes(), n


def test_avg_split_divides_once_in_fp32():
    """n = 72: p = 16, q = 4.5; fp32 values whose sum / 16 is exact: the split
    result is the correctly rounded fp32 quotient of the exact sum by 72."""
    n = 72
    rg = np.random.default_rng(17)
    xs = [(rg.integers(-1000, 1000, size=40) * 16).astype(np.float32) for _ in range(n)]
    got = oracle.ring_allreduce(xs, "f32", "avg", avg_split=True)[0]
    total = sum(x.astype(np.int64) for x in xs)
    want = ((total // 16).astype(np.float32) / np.float32(4.5)).astype(np.float32)
    assert got.tobytes() == want.tobytes()
    i = oracle.ring_allreduce([x.astype(np.int32) for x in xs], "i32", "avg", avg_split=True)[0]
    assert i.tobytes() == oracle.ring_allreduce([x.astype(np.int32) for x in xs], "i32", "avg")[0].tobytes()


# ---------------------------------------------------------------------------
# 7. invariants the pages state
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_allreduce_is_reduce_scatter_then_all_gather(dtype):
    """all-reduce = reduce-scatter + all-gather, bit for bit, when the chunks of
    the two calls coincide (count a multiple of n 16-byte units)."""
    for n in (1, 2, 3, 5, 8):
        u = 16 // workloads.ELEM_SIZE[dtype]
        count = n * u * 7
        for op in OPS:
            xs = [workloads.random_values(13, n, r, count, dtype) for r in range(n)]
            ar = oracle.ring_allreduce(xs, dtype, op)
            ag = oracle.ring_all_gather(oracle.ring_reduce_scatter(xs, dtype, op), dtype)
            for a, b in zip(ar, ag):
                assert a.tobytes() == b.tobytes(), (dtype, n, op)
            for a in ar[1:]:
                assert a.tobytes() == ar[0].tobytes()          # every rank identical


@pytest.mark.parametrize("dtype", DTYPES)
def test_in_place_equals_out_of_place(dtype):
    n, count = 5, 203
    for op in OPS:
        xs = [workloads.random_values(14, 0, r, count, dtype) for r in range(n)]
        ref = oracle.ring_allreduce(xs, dtype, op)
        buf = [x.copy() for x in xs]
        oracle.ring_allreduce(buf, dtype, op, out=buf)
        for a, b in zip(ref, buf):
            assert a.tobytes() == b.tobytes()
        buf = [x.copy() for x in xs]
        oracle.tree_allreduce(buf, dtype, op, out=buf)
        for a, b in zip(oracle.tree_allreduce(xs, dtype, op), buf):
            assert a.tobytes() == b.tobytes()


# ---------------------------------------------------------------------------
# 8. the oracle's own conversions, against library routines
# ---------------------------------------------------------------------------

def _edge_f32():
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e-8, 2.0 ** -24, 2.0 ** -25,
            2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
            float(np.finfo(np.float32).max), float(np.finfo(np.float32).tiny), float("inf"), float("-inf"),
            1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, 256.0 + 1.0, 3.0e38]
    rg = np.random.default_rng(0)
    bits = rg.integers(0, 2 ** 32, size=60000, dtype=np.uint64).astype(np.uint32)
    rnd = bits.view(np.float32)
    rnd = rnd[np.isfinite(rnd)]
    scaled = (rg.standard_normal(60000) * 10.0 ** rg.uniform(-9, 6, 60000)).astype(np.float32)
    return np.concatenate([np.array(vals, np.float32), rnd, scaled])


def test_bf16_rounding_matches_torch():
    import torch
    v = _edge_f32()
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16_bits(float(x)) for x in v], np.uint16)
    assert np.array_equal(got, want)
    back = np.array([oracle.bf16_bits_to_f32(int(h)) for h in want[:5000]], np.float32)
    assert np.array_equal(back.view(np.uint32), want[:5000].astype(np.uint32) << 16)


def test_f16_conversions_match_numpy():
    v = _edge_f32()
    want = v.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_bits(float(x)) for x in v], np.uint16)
    assert np.array_equal(got, want)
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = allh.view(np.float16).astype(np.float32)
    got32 = np.array([oracle.f16_bits_to_f32(int(h)) for h in allh], np.float32)
    finite = np.isfinite(exp)
    assert np.array_equal(got32[finite].view(np.uint32), exp[finite].view(np.uint32))
    assert np.all(np.isnan(got32[np.isnan(exp)]))
