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
    assert _err(ar.ar_allreduce, A[:2], B[:2], 16, "f32", "sum", sched=5) == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_allreduce, [A[0], 0], B[:2], 16, "f32", "sum") == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_allreduce, A[:2], [B[0], 0], 16, "f32", "sum") == "AR_ERR_INVALID_ARG"
    # misaligned for the element size
    assert _err(ar.ar_allreduce, [A[0] + 2, A[1]], B[:2], 16, "f32", "sum") == "AR_ERR_ALIGNMENT"
    assert _err(ar.ar_allreduce, [A[0] + 1, A[1]], B[:2], 16, "bf16", "sum") == "AR_ERR_ALIGNMENT"
    # tree is not a reduce-scatter / all-gather schedule
    assert _err(ar.ar_reduce_scatter, A[:2], B[:2], 16, "f32", "sum", sched="tree") == "AR_ERR_UNSUPPORTED"
    assert _err(ar.ar_all_gather, A[:2], B[:2], 16, "f32", sched="tree") == "AR_ERR_UNSUPPORTED"


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


def test_tree_parent_matches_the_14_rank_picture():
    with open(os.path.join(ROOT, "tests", "golden", "tree14.json")) as f:
        g = json.load(f)
    assert [ar.ar_tree_parent(g["n"], v) for v in range(g["n"])] == g["parent"]
    assert ar.ar_tree_parent(4, 7) == -1 and ar.ar_tree_parent(0, 0) == -1


def test_plan_steps_bytes_and_legality():
    for n in (1, 2, 4, 8, 16, 72, 128):
        count = 1 << 20
        p = ar.ar_plan("allreduce", count, "f32", "sum", n)
        assert p.legal == ["ring", "tree", "fused"]
        assert p.steps["ring"] == 2 * (n - 1)
        assert p.steps["tree"] == 2 * ((n - 1).bit_length() if n > 1 else 0)
        assert p.steps["fused"] == 1
        assert all(b == 2 * n * count * 4 for b in p.bytes.values())
        assert p.chosen == min(p.predicted_us, key=lambda s: (p.predicted_us[s], ar.SCHEDS[s]))
        for coll in ("reduce_scatter", "all_gather"):
            q = ar.ar_plan(coll, count, "bf16", "avg", n)
            assert q.legal == ["ring", "fused"]
            assert q.steps["ring"] == n - 1
            assert all(b == (n + 1) * n * count * 2 for b in q.bytes.values())


def test_plan_is_monotone_in_size():
    prev = None
    for k in range(0, 31, 2):
        p = ar.ar_plan("allreduce", 1 << k, "i32", "sum", 16)
        t = p.predicted_us[p.chosen]
        if prev is not None:
            assert t >= prev
        prev = t


def test_plan_rejects_bad_arguments():
    assert _err(ar.ar_plan, "allreduce", 16, "f32", "sum", 0) == "AR_ERR_INVALID_ARG"
    assert _err(ar.ar_plan, 3, 16, "f32", "sum", 4) == "AR_ERR_INVALID_ARG"
