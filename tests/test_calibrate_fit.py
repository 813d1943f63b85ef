"""The cost-model fit (reduce_scatter_amd/calibrate.py) on synthetic
measurements: it recovers launch, per-step and bandwidth constants, and each
footprint of 1 GB and more keeps its own correction (a schedule that slows
only at the largest footprints is priced slower there, not everywhere)."""
from __future__ import annotations

import math

from reduce_scatter_amd import calibrate as cal


def _rows(slow_big_split):
    rows = []
    for n in (2, 8, 16):
        for k in range(10, 31):
            pr = 1 << k
            for sched, launch, step, bw in (("ring", 7.0, 0.1, 5000.0), ("fused", 8.0, 0.0, 6000.0),
                                            ("split", 8.0, 0.0, 6000.0)):
                b = cal._bytes("allreduce", n, pr)
                eff = bw
                if sched == "split" and slow_big_split and b >= (1 << 34):
                    eff = bw * 0.8                                  # slows past 16 GB of traffic
                us = launch + step * cal._steps("allreduce", sched, n) + b / 1e3 / eff
                rows.append(("allreduce", sched, n, pr, us))
    return rows


def test_fit_recovers_the_constants():
    model = cal.fit(_rows(False))
    launch, step, bw, corr, extra = model[("allreduce", "ring")]
    assert abs(launch - 7.0) < 0.05 and abs(step - 0.1) < 0.005
    assert abs(bw - 5000.0) / 5000.0 < 0.01
    launch, step, bw, corr, extra = model[("allreduce", "fused")]
    assert abs(launch - 8.0) < 0.05 and step == 0.0 and abs(bw - 6000.0) / 6000.0 < 0.01
    for rc, row in corr.items():                                    # no size dependence to correct
        assert all(abs(c - 1.0) < 0.02 for c in row[20:])


def test_large_footprints_keep_their_own_correction():
    model = cal.fit(_rows(True))
    _, _, bw_s, corr_s, _ = model[("allreduce", "split")]
    _, _, bw_f, corr_f, _ = model[("allreduce", "fused")]
    rc = math.ceil(math.log2(16))
    pred = lambda bw, corr, b: b / 1e3 / (bw * corr[rc][int(math.log2(b))])
    small, big = 1 << 31, 1 << 35                                   # 2 GB and 32 GB of traffic at n = 16
    assert pred(bw_s, corr_s, small) <= 1.02 * pred(bw_f, corr_f, small)   # split as fast as fused at 2 GB
    assert pred(bw_s, corr_s, big) >= 1.15 * pred(bw_f, corr_f, big)       # and priced slower at 32 GB


def test_two_byte_fit_keeps_the_latency_terms():
    """The bf16 fit takes launch, step and extra latency from the fp32 fit and
    fits only the bandwidth: a type whose rate differs is priced by its own
    rate with the shared latency model."""
    rows4 = _rows(False)
    model4 = cal.fit(rows4)
    rows2 = [(c, s, n, pr, us + (pr * 2 * n) / 1e3 / 6000.0 * (0.25 if s == "ring" else 0.0))
             for c, s, n, pr, us in rows4]                 # the ring 25 % slower on the bandwidth term
    model2 = cal.fit(rows2, latency=model4)
    for key in model4:
        assert model2[key][0] == model4[key][0] and model2[key][1] == model4[key][1]
        assert model2[key][4] == model4[key][4]
    assert model2[("allreduce", "ring")][2] < model4[("allreduce", "ring")][2]
    assert abs(model2[("allreduce", "fused")][2] - model4[("allreduce", "fused")][2]) / model4[("allreduce", "fused")][2] < 0.01


def test_merge_replaces_only_the_remeasured_schedules(tmp_path):
    """``--schedules S --merge BASE``: the file keeps every entry of BASE whose
    schedule is not in S, takes S's entries from the new fit (dropping BASE's
    lines for S, including rank classes the new fit has none for), and names
    the re-measured schedules in its header."""
    full = cal.fit(_rows(False))
    base_path = tmp_path / "base.txt"
    cal.write(str(base_path), full, "box A")
    base = cal.read_entries(str(base_path))
    rows = [(c, s, n, pr, us * 1.5) for c, s, n, pr, us in _rows(False) if s == "ring"]
    part = cal.fit(rows)
    assert {k[1] for k in part} == {"ring"}
    out = tmp_path / "merged.txt"
    cal.write(str(out), part, "box B", base=base, scheds=("ring", "tree"))
    header, entries = cal.read_entries(str(out))
    assert "# device: box A" in header and "# re-measured: ring, tree on box B" in header
    assert set(entries) == set(base[1])
    for key, lines in entries.items():
        if key[1] == "ring":
            assert lines == cal.entry_lines(part)[key] and lines != base[1][key]
        else:
            assert lines == base[1][key]


def test_merge_by_rank_class_keeps_the_base_constants(tmp_path):
    """``--ranks``: the re-measured schedule keeps BASE's launch, step and
    bandwidth line and its other rank classes; only the named classes' rows
    are replaced, fitted relative to BASE's bandwidth (a 1.5x slower
    re-measurement at 16 ranks shows as corrections near 1/1.5 there)."""
    full = cal.fit(_rows(False))
    base_path = tmp_path / "base.txt"
    cal.write(str(base_path), full, "box A")
    base = cal.read_entries(str(base_path))
    fixed, _ = cal.base_constants(base)
    assert fixed[("allreduce", "ring")] == tuple(float(x) for x in base[1][("allreduce", "ring")][0].split()[2:5])
    rows = [(c, s, n, pr, us * 1.5) for c, s, n, pr, us in _rows(False) if s == "ring" and n == 16]
    part = cal.fit(rows, fixed=fixed)
    out = tmp_path / "merged.txt"
    cal.write(str(out), part, "box B", base=base, scheds=("ring",), classes={4})
    header, entries = cal.read_entries(str(out))
    assert "# re-measured: ring for rank classes 4 on box B" in header
    ring, old = entries[("allreduce", "ring")], base[1][("allreduce", "ring")]
    assert ring[0] == old[0]                                        # launch, step, bandwidth kept
    assert [l for l in ring if cal._row_class(l) in (1, 3)] == [l for l in old if cal._row_class(l) in (1, 3)]
    new4 = [l for l in ring if l.startswith("corr ") and cal._row_class(l) == 4]
    assert len(new4) == 1
    big = [float(x) for x in new4[0].split()[4:]][32:]             # footprints of 4 GB and more
    assert all(abs(c - 1 / 1.5) < 0.05 for c in big)
    for key, lines in entries.items():
        if key[1] != "ring":
            assert lines == base[1][key]
