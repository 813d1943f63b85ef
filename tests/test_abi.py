"""The C ABI without a GPU: exported symbols, argument validation (which
happens before any HIP call), the cost model and the tree builder."""
from __future__ import annotations

import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ar.h")

ar = pytest.importorskip("reduce_scatter_amd", reason="libar.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ar_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"ar_allreduce", "ar_reduce_scatter", "ar_all_gather", "ar_plan"} <= set(names)
    lib = ctypes.CDLL(ar.library_path())
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    for code, name in ((0, "AR_OK"), (1, "AR_ERR_INVALID_ARG"), (2, "AR_ERR_UNSUPPORTED"), (3, "AR_ERR_ALIGNMENT"),
                       (4, "AR_ERR_HIP")):
        assert ar.ar_status_string(code).startswith(name)


def _err(fn, *a, **k):
    with pytest.raises(ar.ArError) as e:
        fn(*a, **k)
    return e.value.name


# Fake, well-aligned, non-overlapping device addresses: validation rejects
# the bad calls below before anything touches a device.
A = [1 << 20, 2 << 20, 3 << 20, 4 << 20]
B = [5 << 20, 6 << 20, 7 << 20, 8 << 20]


def test_invalid_arguments_are_rejected_before_launch():
    assert _err(ar.ar_allreduce, A[:2], B[:2], 16, "f32", "sum", n=0) == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_allreduce, A[:2], B[:2], 16, "f32", "sum", n=129) == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_allreduce, A[:2], B[:2], 16, 7, "sum") == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_allreduce, A[:2], B[:2], 16, "f32", 9) == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_allreduce, A[:2], B[:2], 16, "f32", "sum", sched=6) == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_allreduce, [A[0], 0], B[:2], 16, "f32", "sum") == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_allreduce, A[:2], [B[0], 0], 16, "f32", "sum") == "AR_ERR_INVALID_ARG"
    # misaligned for the element size
    assert _err(ar.ar_allreduce, [A[0] + 2, A[1]], B[:2], 16, "f32", "sum") == "AR_ERR_ALIGNMENT"
    assert _err(ar.ar_allreduce, [A[0] + 1, A[1]], B[:2], 16, "bf16", "sum") == "AR_ERR_ALIGNMENT"
    # tree and split are all-reduce schedules only
    for sched in ("tree", "split", "dtree"):
        assert _err(ar.ar_reduce_scatter, A[:2], B[:2], 16, "f32", "sum", sched=sched) == "AR_ERR_UNSUPPORTED"
        assert _err(ar.ar_all_gather, A[:2], B[:2], 16, "f32", sched=sched) == "AR_ERR_UNSUPPORTED"


def test_numerics_are_validated_before_launch():
    bad = [("acc", 2), ("avg", 7), ("acc", -1)]
    for field, value in bad:
        kw = {"acc": "storage", "avg": "prescale"}
        kw[field] = value
        assert _err(ar.ar_allreduce_ex, A[:2], B[:2], 64, "bf16", "avg", **kw) == "AR_ERR_INVALID_ARG"
        assert _err(ar.ar_reduce_scatter_ex, A[:2], B[:2], 64, "bf16", "avg", **kw) == "AR_ERR_INVALID_ARG"
    # fp32 partials for bf16 / fp16 exist on the fused schedule only
    for dtype in ("bf16", "f16"):
        for sched in ("ring", "tree", "split", "dtree"):
            assert _err(ar.ar_allreduce_ex, A[:2], B[:2], 64, dtype, "sum", sched=sched, acc="fp32") == \
                "AR_ERR_UNSUPPORTED"
        assert _err(ar.ar_reduce_scatter_ex, A[:2], B[:2], 64, dtype, "sum", sched="ring", acc="fp32") == \
            "AR_ERR_UNSUPPORTED"


def test_zero_count_is_a_no_op():
    ar.ar_allreduce(A[:2], B[:2], 0, "f32", "sum")
    ar.ar_reduce_scatter(A[:2], B[:2], 0, "bf16", "avg")
    ar.ar_all_gather(A[:2], B[:2], 0, "i32")


def test_overlap_rules():
    S = 1024 * 4                                    # 1024 fp32
    # recv overlapping another rank's send buffer
    assert _err(ar.ar_allreduce, A[:2], [A[1], B[1]], 1024, "f32", "sum") == "AR_ERR_INVALID_ARG"
    # recv partially overlapping its own send buffer (not the in-place layout)
    assert _err(ar.ar_allreduce, A[:2], [A[0] + 16, B[1]], 1024, "f32", "sum") == "AR_ERR_INVALID_ARG"
    # two recv buffers overlapping
    assert _err(ar.ar_allreduce, A[:2], [B[0], B[0] + S - 16], 1024, "f32", "sum") == "AR_ERR_INVALID_ARG"
    # aliased send buffers with one of them written in place
    assert _err(ar.ar_allreduce, [A[0], A[0]], [A[0], B[1]], 1024, "f32", "sum") == "AR_ERR_INVALID_ARG"
    # reduce-scatter: in place means recv[r] = send[r] + r*R elements; anything else that overlaps fails
    R = 256
    assert _err(ar.ar_reduce_scatter, A[:2], [A[0] + 16, B[1]], R, "f32", "sum") == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_reduce_scatter, A[:2], [A[0] + R * 4, B[1]], R, "f32", "sum") == "AR_ERR_INVALID_ARG"
    # all-gather: in place means send[r] = recv[r] + r*R elements
    assert _err(ar.ar_all_gather, [B[0] + 16, A[1]], B[:2], R, "f32") == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_all_gather, [B[1], A[1]], B[:2], R, "f32") == "AR_ERR_INVALID_ARG"


def _brute_conflict(send, slen, recv, rlen, allowed):
    """Pairwise rule: a recv range may overlap nothing but its own send range in
    the allowed in-place layout; send ranges may overlap each other."""
    ov = lambda a, al, b, bl: a < b + bl and b < a + al
    n = len(send)
    for r in range(n):
        for k in range(n):
            if ov(recv[r], rlen, send[k], slen) and not (k == r and allowed[r]):
                return True
        for k in range(r + 1, n):
            if ov(recv[r], rlen, recv[k], rlen):
                return True
    return False


def test_overlap_check_matches_the_pairwise_rule():
    """Random layouts on a coarse address grid (overlaps are frequent): the
    library rejects exactly the layouts the pairwise rule rejects; accepted
    layouts get as far as the device query, which fails without a GPU."""
    import random
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("host-logic test: an accepted layout would launch on addresses nobody owns")
    rng = random.Random(5)
    base = 1 << 32
    unit = 256                                            # bytes: 64 fp32
    for trial in range(3000):
        n = rng.randint(1, 9)
        coll = rng.choice(["allreduce", "reduce_scatter", "all_gather"])
        R = 64                                            # elements per slice
        if coll == "allreduce":
            slen = rlen = R * 4
        elif coll == "reduce_scatter":
            slen, rlen = n * R * 4, R * 4
        else:
            slen, rlen = R * 4, n * R * 4
        span = 4 * n * max(slen, rlen) // unit
        send = [base + unit * rng.randrange(span) for _ in range(n)]
        recv = [base + unit * rng.randrange(span) for _ in range(n)]
        for r in range(n):                                # make some ranks use the in-place layout
            if rng.random() < 0.3:
                if coll == "allreduce":
                    recv[r] = send[r]
                elif coll == "reduce_scatter":
                    recv[r] = send[r] + r * R * 4
                else:
                    send[r] = recv[r] + r * R * 4
        if coll == "allreduce":
            allowed = [recv[r] == send[r] for r in range(n)]
            call = lambda: ar.ar_allreduce(send, recv, R, "f32", "sum", sched="fused")
        elif coll == "reduce_scatter":
            allowed = [recv[r] == send[r] + r * R * 4 for r in range(n)]
            call = lambda: ar.ar_reduce_scatter(send, recv, R, "f32", "sum", sched="fused")
        else:
            allowed = [send[r] == recv[r] + r * R * 4 for r in range(n)]
            call = lambda: ar.ar_all_gather(send, recv, R, "f32", sched="fused")
        want = _brute_conflict(send, slen, recv, rlen, allowed)
        got = _err(call) == "AR_ERR_INVALID_ARG"
        assert got == want, (trial, coll, n, send, recv)


def test_tree_parent_matches_the_14_rank_picture():
    with open(os.path.join(ROOT, "tests", "golden", "tree14.json")) as f:
        g = json.load(f)
    assert [ar.ar_tree_parent(g["n"], v) for v in range(g["n"])] == g["parent"]
    assert ar.ar_tree_parent(4, 7) == -1 and ar.ar_tree_parent(0, 0) == -1


def test_dtree_parent_is_the_complementary_tree():
    """The second tree: the mirror image of the first for even n, the first
    shifted by one rank for odd n; the first is ar_tree_parent's tree."""
    def first(n, v):
        if v == 0:
            return -1
        b = v & -v
        p = (v ^ b) | (b << 1)
        return v ^ b if p >= n else p
    for n in range(1, 129):
        for v in range(n):
            assert ar.ar_dtree_parent(n, 0, v) == ar.ar_tree_parent(n, v) == first(n, v)
            if n % 2 == 0:
                q = first(n, n - 1 - v)
                want = -1 if q < 0 else n - 1 - q
            else:
                q = first(n, (v - 1) % n)
                want = -1 if q < 0 else (q + 1) % n
            assert ar.ar_dtree_parent(n, 1, v) == want, (n, v)
    assert ar.ar_dtree_parent(8, 2, 1) == -1 and ar.ar_dtree_parent(8, 1, 8) == -1


def _expected_choice(pred, footprint, n):
    """The cost model's choice: the least predicted time (ties to the lower
    schedule code), except that the preferred schedule (split past 16 ranks
    where legal, else fused) is kept within 0.5 us of the least, and for
    footprints of 1 GB and more within 3 %."""
    best = min(pred, key=lambda s: (pred[s], ar.SCHEDS[s]))
    pref = "split" if n > 16 and "split" in pred else "fused"
    if pref in pred and (pred[pref] <= pred[best] + 0.5 or
                         (footprint >= (1 << 30) and pred[pref] <= pred[best] * 1.03)):
        return pref
    return best


def test_plan_steps_bytes_and_legality():
    for n in (1, 2, 4, 8, 16, 72, 128):
        count = 1 << 20
        p = ar.ar_plan("allreduce", count, "f32", "sum", n)
        assert p.legal == ["ring", "tree", "fused", "split", "dtree"]
        assert p.steps["ring"] == 2 * (n - 1)
        assert p.steps["tree"] == 2 * ((n - 1).bit_length() if n > 1 else 0)
        assert p.steps["fused"] == 1 and p.steps["split"] == 1
        assert p.steps["dtree"] == p.steps["tree"]
        assert all(b == 2 * n * count * 4 for b in p.bytes.values())
        assert p.chosen == _expected_choice(p.predicted_us, max(p.bytes.values()), n)
        for coll in ("reduce_scatter", "all_gather"):
            q = ar.ar_plan(coll, count, "bf16", "avg", n)
            assert q.legal == ["ring", "fused"]
            assert q.steps["ring"] == n - 1
            assert all(b == (n + 1) * n * count * 2 for b in q.bytes.values())


def _plan_in_subprocess(calib, calls):
    """Run ar_plan in a fresh process (the calibration file is read once per process)."""
    import subprocess
    import sys
    code = "import json, sys; sys.path.insert(0, %r); import reduce_scatter_amd as ar; " \
           "print(json.dumps([ar.ar_plan(*c).__dict__ for c in %r]))" % (ROOT, calls)
    env = dict(os.environ, AR_CALIB=calib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_plan_is_monotone_in_size_with_default_constants():
    calls = [("allreduce", 1 << k, "i32", "sum", 16) for k in range(0, 31, 2)]
    plans = _plan_in_subprocess("/nonexistent/calib.txt", calls)
    times = [p["predicted_us"][p["chosen"]] for p in plans]
    assert times == sorted(times)


def test_plan_rank_classes_split_the_top_octave(tmp_path):
    """Rank class ceil(log2 n), except 97-128 ranks (class 8) apart from 65-96
    (class 7): each takes its own correction row, and a class with no row
    takes the nearest measured one.  The latency term likewise: a class the
    file measured (a lat or corr row) takes its own, zero without a lat row;
    a class it did not measure takes the nearest measured class's."""
    f = tmp_path / "classes.txt"
    half = " ".join(["0.5"] * 48)
    one = " ".join(["1.0"] * 48)
    f.write_text("allreduce fused 10 0 1000\nallreduce split 10 0 1000\nallreduce ring 1000 0 1000\n"
                 "allreduce tree 1000 0 1000\nallreduce dtree 1000 0 1000\n"
                 "corr allreduce fused 7 " + one + "\ncorr allreduce fused 8 " + half + "\n"
                 "corr allreduce split 5 " + one + "\nlat allreduce split 5 3.0\n"
                 "corr allreduce split 7 " + one + "\n")
    count = 1 << 16
    calls = [("allreduce", count, "f32", "sum", n) for n in (72, 96, 97, 128, 40, 33)]
    p72, p96, p97, p128, p40, p33 = _plan_in_subprocess(str(f), calls)
    for p, n in ((p72, 72), (p96, 96), (p97, 97), (p128, 128)):
        b = 2 * n * count * 4
        corr = 0.5 if n > 96 else 1.0
        assert abs(p["predicted_us"]["fused"] - (10 + b / 1e3 / (1000 * corr))) < 1e-6, n
        assert abs(p["predicted_us"]["split"] - (10 + b / 1e3 / 1000)) < 1e-6, n    # class 7 measured, no lat row
    for p, n in ((p40, 40), (p33, 33)):                         # class 6: no row; split's nearest is class 5
        b = 2 * n * count * 4
        assert abs(p["predicted_us"]["split"] - (10 + 3.0 + b / 1e3 / 1000)) < 1e-6, n


def test_plan_reads_the_calibration_file(tmp_path):
    """Constants and the (rank class x footprint) correction come from the file:
    t = launch + step * steps + bytes / (bw * corr)."""
    f = tmp_path / "calib.txt"
    corr = ["1.0"] * 48
    corr[27] = "0.5"                     # 2^27 .. 2^28 - 1 bytes in total
    f.write_text("allreduce ring 10 0.5 1000\nallreduce tree 20 1 1000\nallreduce fused 5 0 500\n"
                 "allreduce split 7 0 400\nlat allreduce split 3 2.5\n"
                 "corr allreduce fused 3 " + " ".join(corr) + "\n")
    count = (1 << 27) // (2 * 8 * 4)     # n = 8 fp32: 2*n*S = 2^27 bytes
    p = _plan_in_subprocess(str(f), [("allreduce", count, "f32", "sum", 8)])[0]
    b = 2 * 8 * count * 4
    assert abs(p["predicted_us"]["ring"] - (10 + 0.5 * 14 + b / 1e3 / 1000)) < 1e-6
    assert abs(p["predicted_us"]["tree"] - (20 + 1 * 6 + b / 1e3 / 1000)) < 1e-6
    assert abs(p["predicted_us"]["fused"] - (5 + b / 1e3 / (500 * 0.5))) < 1e-6
    assert abs(p["predicted_us"]["split"] - (7 + 2.5 + b / 1e3 / 400)) < 1e-6
    assert p["chosen"] == _expected_choice(p["predicted_us"], b, 8)
    # the tie margin, for calls that stream from HBM (footprint >= 1 GB): fused within 3 % of a faster
    # prediction keeps the call, beyond it does not; below 1 GB the argmin stands
    g = tmp_path / "tie.txt"
    g.write_text("allreduce ring 1000 0 1000\nallreduce tree 1000 0 1000\nallreduce split 1000 0 1000\n"
                 "allreduce dtree 0 0 1000\nallreduce fused 10 0 1000\n")
    big = (1 << 30) // (2 * 8 * 4)       # n = 8 fp32: a 1 GB footprint
    near, far, cache = _plan_in_subprocess(str(g), [("allreduce", big, "f32", "sum", 8),
                                                    ("allreduce", big // 64, "f32", "sum", 8),
                                                    ("allreduce", big // 2, "f32", "sum", 8)])
    assert near["chosen"] == "fused" and near["predicted_us"]["dtree"] < near["predicted_us"]["fused"]
    assert near["predicted_us"]["fused"] <= 1.03 * near["predicted_us"]["dtree"]
    assert far["chosen"] == "dtree" and far["predicted_us"]["fused"] > 1.03 * far["predicted_us"]["dtree"]
    assert cache["predicted_us"]["fused"] <= 1.03 * cache["predicted_us"]["dtree"] and cache["chosen"] == "dtree"
    # past 16 ranks split is the schedule the margin keeps: fused predicted 2 % faster than split at 72 ranks
    h = tmp_path / "tie72.txt"
    h.write_text("allreduce ring 1000 0 1000\nallreduce tree 1000 0 1000\nallreduce dtree 1000 0 1000\n"
                 "allreduce fused 0 0 1000\nallreduce split 0 0 980\n")
    c72 = (1 << 30) // (2 * 72 * 4) + 64   # n = 72 fp32: a footprint just over 1 GB
    p72, p8 = _plan_in_subprocess(str(h), [("allreduce", c72, "f32", "avg", 72), ("allreduce", big, "f32", "sum", 8)])
    assert p72["predicted_us"]["fused"] < p72["predicted_us"]["split"] <= 1.03 * p72["predicted_us"]["fused"]
    assert p72["chosen"] == "split" and p8["chosen"] == "fused"
    assert p72["chosen"] == _expected_choice(p72["predicted_us"], max(p72["bytes"].values()), 72)
    # a rank class with no row of its own uses the nearest measured one (class 3 for n = 16)
    p16 = _plan_in_subprocess(str(f), [("allreduce", count // 2, "f32", "sum", 16)])[0]
    assert abs(p16["predicted_us"]["fused"] - (5 + b / 1e3 / (500 * 0.5))) < 1e-6


def test_plan_uses_the_two_byte_tables_for_bf16_and_fp16(tmp_path):
    """bw2 / corr2 records price the 2-byte types; 4-byte types keep the main
    tables, and a schedule without a 2-byte rate falls back to them."""
    f = tmp_path / "calib.txt"
    corr2 = ["1.0"] * 48
    corr2[27] = "0.25"
    f.write_text("allreduce ring 10 0 1000\nallreduce fused 5 0 1000\nallreduce split 7 0 1000\n"
                 "allreduce tree 9 0 1000\nallreduce dtree 9 0 1000\n"
                 "bw2 allreduce fused 2000\ncorr2 allreduce fused 3 " + " ".join(corr2) + "\n"
                 "bw2 allreduce ring 500\n")
    b = 1 << 27                                   # 2*n*S at n = 8 for every dtype below
    calls = [("allreduce", b // (2 * 8 * e), dt, "sum", 8) for dt, e in (("f32", 4), ("i32", 4), ("bf16", 2), ("f16", 2))]
    p32, pi32, pbf, pf16 = _plan_in_subprocess(str(f), calls)
    for p in (p32, pi32):
        assert abs(p["predicted_us"]["fused"] - (5 + b / 1e3 / 1000)) < 1e-6
        assert abs(p["predicted_us"]["ring"] - (10 + b / 1e3 / 1000)) < 1e-6
    for p in (pbf, pf16):
        assert abs(p["predicted_us"]["fused"] - (5 + b / 1e3 / (2000 * 0.25))) < 1e-6
        # a 2-byte rate without a 2-byte correction row takes the 4-byte one (none here: all ones)
        assert abs(p["predicted_us"]["ring"] - (10 + b / 1e3 / 500)) < 1e-6
        # no 2-byte record at all: the 4-byte table
        assert abs(p["predicted_us"]["split"] - (7 + b / 1e3 / 1000)) < 1e-6


def test_plan_rejects_bad_arguments():
    assert _err(ar.ar_plan, "allreduce", 16, "f32", "sum", 0) == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_plan, 3, 16, "f32", "sum", 4) == "AR_ERR_INVALID_ARG"
