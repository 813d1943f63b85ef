"""Planted mistakes in the oracle, each caught by a pin.  CPU only.

Every case below copies ``oracle/ar_oracle.c``, plants one plausible mistake
by text substitution (a ceiling instead of a floor in the chunk cut, a
per-contribution divide instead of the pre-scale, a wrong chunk index, a
dropped step, a flipped tie rule, ...), builds the copy with gcc into a
temporary directory, points the ``oracle`` wrapper at it, and runs the pins
named for that mistake: at least one of them must fail.  A control build of
the unchanged source must pass every pin, so a failure comes from the planted
mistake and not from the build.

Every mutant keeps the oracle's memory accesses in bounds (the wire buffers
hold the longest chunk), so a planted mistake changes values, never crashes
the test process.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import pytest

import oracle
import test_brute as TB
import test_oracle as T

SRC = os.path.join(os.path.dirname(oracle.__file__), "ar_oracle.c")


def pins_avg_prescale():
    for case in T.PRESCALE_CASES:
        yield lambda case=case: T.test_float_avg_prescale_hand_cases(*case)


# (name, [(old text, new text, occurrences to replace or 0 for all)], pins that must catch it)
MUTANTS = [
    ("ceiling chunk cut",
     [("((unsigned __int128)c * V) / (unsigned)n", "((unsigned __int128)c * V + (unsigned)n - 1) / (unsigned)n", 0)],
     [T.test_allreduce_chunks_floor_cut_hand_cases, lambda: T.test_floor_cut_decides_the_hop_order_of_the_cut_vectors("f32")]),
    ("float avg as a per-contribution divide by n",
     [("own.f = own.f * s;", "own.f = own.f / (float)(int)(1.0f / s + 0.5f);", 0)],
     list(pins_avg_prescale())),
    ("float avg as sum, then one divide by n",
     [("if (op == ORC_AVG && dtype != ORC_I32) own.f = own.f * s;", "(void)s;", 0),
      ("if (op == ORC_AVG && dtype == ORC_I32) acc.u = (uint32_t)((int32_t)acc.u / (int32_t)n);",
       "if (op == ORC_AVG && dtype == ORC_I32) acc.u = (uint32_t)((int32_t)acc.u / (int32_t)n);"
       " else if (op == ORC_AVG) acc.f = acc.f / (float)n;", 0)],
     list(pins_avg_prescale())),
    ("chain starting at the owner (rank r sends chunk r first)",
     [("int c = mod_n((long long)r - 1 - t, n);\n            size_t len = off[c + 1] - off[c];\n            const void *mine",
       "int c = mod_n((long long)r - t, n);\n            size_t len = off[c + 1] - off[c];\n            const void *mine", 1)],
     [lambda: T.test_ring_hop_order_rounding_cases("f32")]),
    ("avg pre-scale applied twice",
     [("own.f = own.f * s;", "own.f = (own.f * s) * s;", 0)],
     [lambda: T.test_worked_example_reduce_scatter_avg("f32")]),
    ("min keeps the own value on ties",
     [("(own.f < acc.f) ? own.f : acc.f", "(own.f <= acc.f) ? own.f : acc.f", 0)],
     [T.test_min_max_ties_keep_incoming]),
    ("bf16 partials not rounded at each hop",
     [("if (dtype == ORC_BF16) v.f = bf16_to_f32(f32_to_bf16(v.f));", "if (dtype == -1) v.f = 0;", 0),
      ("case ORC_BF16: ((uint16_t *)buf)[i] = f32_to_bf16(v.f); break;",
       "case ORC_BF16: ((uint16_t *)buf)[i] = f32_to_bf16(v.f); break; /* rounded only when stored */", 0)],
     [T.test_bf16_rounds_at_every_hop]),
    ("tree children in descending rank order",
     [("for (int ch = 0; ch < n; ++ch)                       /* children may rank below or above v */",
       "for (int ch = n - 1; ch >= 0; --ch)", 0)],
     [T.test_tree_order_own_first_then_children_ascending]),
    ("integer avg floors instead of truncating",
     [("acc.u = (uint32_t)((int32_t)acc.u / (int32_t)n);",
       "acc.u = (uint32_t)(((int32_t)acc.u - (((int32_t)acc.u % (int32_t)n) < 0 ? (int32_t)n + ((int32_t)acc.u % (int32_t)n) : ((int32_t)acc.u % (int32_t)n))) / (int32_t)n);", 0)],
     [lambda: T.test_brute_force_allreduce("i32", "avg")]),
    ("one reduce step dropped",
     [("    for (int t = 0; t <= n - 2; ++t) {\n        for (int r = 0; r < n; ++r) {\n            int c = mod_n((long long)r - 1 - t, n);",
       "    for (int t = 0; t < n - 2; ++t) {\n        for (int r = 0; r < n; ++r) {\n            int c = mod_n((long long)r - 1 - t, n);", 1)],
     [lambda: T.test_brute_force_allreduce("f32", "sum")]),
    ("sum subtracts",
     [("case ORC_SUM: case ORC_AVG: r.f = acc.f + own.f; break;", "case ORC_SUM: case ORC_AVG: r.f = acc.f - own.f; break;", 0)],
     [lambda: T.test_worked_example_allreduce_sum("f32")]),
    ("fp16 ties rounded away from zero",
     [("if (rem > half || (rem == half && (kept & 1u))) kept += 1u;", "if (rem >= half) kept += 1u;", 0)],
     [T.test_f16_conversions_match_numpy]),
    ("bf16 ties rounded away from zero",
     [("if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))", "if (lower >= 0x8000u)", 0)],
     [T.test_bf16_rounding_matches_torch]),
    ("all-gather stores a received chunk at the wrong place",
     [("int c = mod_n((long long)r - 1 - t, n);       /* chunk rank r just received */",
       "int c = mod_n((long long)r - t, n);", 0)],
     [lambda: T.test_worked_example_all_gather("f32"), lambda: TB.test_reduce_scatter_and_all_gather_match_the_brute_evaluation("f32", "sum")]),
    ("tree parent falls back to the root",
     [("if (p >= n) p = v ^ b;                                 /* fallback at the edge of the range */",
       "if (p >= n) p = 0;", 0)],
     [T.test_tree_matches_the_14_rank_picture]),
    ("odd double tree shifted the other way",
     [("int p = orc_tree_parent(n, (v - 1 + n) % n);\n    return p < 0 ? -1 : (p + 1) % n;",
       "int p = orc_tree_parent(n, (v + 1) % n);\n    return p < 0 ? -1 : (p - 1 + n) % n;", 0)],
     [T.test_dtree_parents_follow_the_construction]),
    ("double tree halves rounded up",
     [("const size_t half = u * (V / 2);", "const size_t half = u * ((V + 1) / 2);", 0)],
     [lambda: T.test_dtree_rounding_cases_on_both_halves("f32")]),
    ("pairwise order split in halves instead of powers of two",
     [("while (2 * h < len) h *= 2;                            /* largest power of two below len */",
       "h = len / 2;", 0)],
     [lambda: T.test_pairwise_rounding_cases("f32")]),
    ("fp32 partials option ignored",
     [("return nm->acc32 ? v : round_to_type(dtype, v);", "return round_to_type(dtype, v);", 0)],
     [lambda: T.test_acc32_keeps_what_per_hop_rounding_loses("bf16")]),
    ("split divisor one power of two too large",
     [("while (p * p < n) p *= 2;", "while (p * p <= n) p *= 2;", 0)],
     [T.test_split_p_is_the_power_of_two_nearest_above_sqrt_n]),
]


def _build(tmp_path, name, edits):
    src = open(SRC).read()
    for old, new, times in edits:
        found = src.count(old)
        assert found >= 1, "%s: the text to replace is not in the oracle source any more: %r" % (name, old[:60])
        src = src.replace(old, new, times if times else -1)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(src)
    subprocess.run(["gcc", "-O1", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-w",
                    "-shared", "-fPIC", str(c_path), "-o", str(so_path)], check=True)
    return oracle._bind(ctypes.CDLL(str(so_path)))


def _fails(pin) -> bool:
    try:
        pin()
    except AssertionError:
        return True
    return False


def test_control_build_passes_every_pin(tmp_path, monkeypatch):
    monkeypatch.setattr(oracle, "_lib", _build(tmp_path, "control", []))
    for name, _, pins in MUTANTS:
        for pin in pins:
            assert not _fails(pin), "the unchanged oracle fails a pin named for %r" % name


@pytest.mark.parametrize("name,edits,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name, edits, pins):
    monkeypatch.setattr(oracle, "_lib", _build(tmp_path, name, edits))
    caught = [_fails(pin) for pin in pins]
    assert any(caught), "no pin catches the planted mistake %r" % name
    if name in ("ceiling chunk cut", "float avg as a per-contribution divide by n", "float avg as sum, then one divide by n"):
        assert all(caught), "each of these pins must catch %r on its own: %s" % (name, caught)
