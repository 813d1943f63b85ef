"""Host model of the phased reduce-scatter / all-gather index arithmetic.

Slices whose byte length is not a multiple of 16 go through the phased
kernels (fused_phase.hip) plus the element-wise edge kernels (elem.hip).  This
file restates their index arithmetic in numpy -- the tile grid
(``aligned_tile`` / ``aligned_tiles`` / ``tile_lane``), the two aligned loads
per lane with the clamp of the second one, the funnel shift's byte window and
the element ranges the edge kernels take -- and checks, for every rank count,
element size, input and output phase, slice lengths around tile boundaries
and one, two or four vectors per lane, that

* every load stays inside the 16-byte blocks that hold the rank's input bytes
  (the reduce-scatter's word-aligned form: inside the 4-byte words that hold
  them, each load at a word-aligned address);
* the 16 bytes a lane assembles are exactly the input bytes of the element
  positions of the output vector it writes (so the clamp never changes a
  second vector that the shift uses);
* the phased vectors and the element-wise ranges write every output element
  exactly once, and nothing outside the output.

It models the kernels' arithmetic (no GPU, no oracle); the GPU parity tests
check the values.
"""
import random

import numpy as np
import pytest

TILE = 64                     # one wavefront's vectors per run


def aligned_tile(lo, hi, j, ref, T):
    a = (ref + lo) & (T - 1)
    start = lo - a + j * T
    return start, max(start, lo), min(start + T, hi)


def aligned_tiles(length, T):
    return (length + T - 1) // T + 1 if length > 0 else 0


def lanes(start, lo, hi, U):
    """Byte offsets from the tile's first in-range vector and the in-range flags of all 64*U lanes."""
    v = start + np.arange(TILE * U, dtype=np.int64)
    ok = (v >= lo) & (v < hi)
    c = np.clip(v, lo, hi - 1)
    return (c - lo) * 16, ok


def library_u(n, coll="rs"):
    """Vectors per lane the library's phased kernels take: the reduce-scatter two up to 8 ranks, the
    all-gather two from 2 ranks on."""
    if coll == "ag":
        return 2 if n >= 2 else 1
    return 2 if 2 <= n <= 8 else 1


def rs_words_loads(a, off, whole, U):
    """The word-aligned form's reads for one tile (a = the tile's first input byte, off = the lanes' byte
    offsets): the 16-byte loads' starts, the starts of the words after them that the shift takes
    (none when a is a whole word), and whether each of those words comes from another lane's load
    (whole tiles: lane l + 1's first word, lane 63's from lane 0 of the next run) or is loaded."""
    w, b = a & ~3, a & 3
    loads = w + off
    if b == 0:
        return loads, None
    nxt = w + off + 16
    if whole:
        starts = set((w + off).tolist())
        from_lanes = np.array([x in starts for x in nxt.tolist()])
        # only the last run's lane 63 lies past the tile: one more word load at the tile's end
        assert (nxt[~from_lanes] == w + TILE * U * 16).all() and (~from_lanes).sum() == 1
    return loads, nxt


def emulate_rs(n, e, R, ps, pr, U, refs, slack=0, edge_shift=0, words=False, shift_mask=3):
    """One phased reduce-scatter call; returns the write count of every output element, per rank.
    ``words`` models the word-aligned form (one load per lane from the word at or below its first input
    byte, the next word only for a phase that is not a whole word).  ``slack``, ``edge_shift`` and
    ``shift_mask`` plant mistakes (a clamp that many bytes short, the edge kernel's upper range moved
    that many elements, the shift taken from the 16-byte phase instead of the word phase) for the test
    that the model notices them."""
    Rb = R * e
    writes = np.zeros((n, R), dtype=np.int64)
    head = (16 - pr) // e if pr > 0 else 0
    if head >= R:                                    # all element-wise
        writes += 1
        return writes
    out_off = head * e
    in_off = ps + out_off
    Rv = (Rb - out_off) // 16
    last_off = ((ps + n * Rb - 1) >> 4) << 4
    for c in range(n):
        for j in range(aligned_tiles(Rv, TILE * U)):
            start, lo, hi = aligned_tile(0, Rv, j, refs[c], TILE * U)
            if lo >= hi:
                continue
            off, ok = lanes(start, lo, hi, U)
            a = in_off + c * Rb + lo * 16
            if words:
                # every read inside the words [ps & ~3, end rounded up to a word) holding the input bytes
                wlo, whi = ps & ~3, (ps + n * Rb + 3) & ~3
                loads, nxt = rs_words_loads(a, off, lo == start and hi == start + TILE * U, U)
                assert (loads % 4 == 0).all()
                assert loads.min() >= wlo and (loads + 16).max() <= whi, (n, e, R, ps, pr, U, c, j)
                if nxt is not None:
                    assert nxt.min() >= wlo and (nxt + 4).max() <= whi, (n, e, R, ps, pr, U, c, j)
                    assert np.array_equal(nxt[ok], loads[ok] + 16)
                # the lane's 16 bytes start b bytes into its load: the input of its output vector
                o = lo + off[ok] // 16
                assert np.array_equal(loads[ok] + (a & shift_mask), ps + c * Rb + out_off + 16 * o)
                for q in o:
                    first = (out_off + 16 * int(q)) // e
                    assert first + 16 // e <= R
                    writes[c, first:first + 16 // e] += 1
                continue
            base, ph = a & ~15, a & 15
            rel = last_off - base - slack
            if rel >= 16 * (TILE * U + 1):
                hi_off = off + 16
            else:
                hi_off = np.where(off + 16 < rel, off + 16, rel)
            # both loads inside the blocks [0, last_off + 16) that hold the input bytes [ps, ps + n*Rb)
            for ld in (base + off, base + hi_off):
                assert ld.min() >= 0 and (ld + 16).max() <= last_off + 16, (n, e, R, ps, pr, U, c, j)
            # the assembled window [a + off, a + off + 16) is the input of the lane's output vector
            o = lo + off[ok] // 16
            want = ps + c * Rb + out_off + 16 * o
            assert np.array_equal(a + off[ok], want)
            assert want.min() >= ps and (want + 16).max() <= ps + n * Rb
            if ph:
                assert np.array_equal(hi_off[ok], off[ok] + 16), (n, e, R, ps, pr, U, c, j)
            # the written output bytes [out_off + 16*o, +16), in elements
            for q in o:
                first = (out_off + 16 * int(q)) // e
                assert first + 16 // e <= R
                writes[c, first:first + 16 // e] += 1
    a_, b_ = head, head + Rv * (16 // e) + edge_shift   # the edge kernel takes [0, a) and [b, R)
    writes[:, :a_] += 1
    writes[:, b_:] += 1
    return writes


def emulate_ag(n, e, R, ps, pr, U, ref):
    """One phased all-gather call; returns the write count of every output element (the same on every rank)."""
    Rb = R * e
    writes = np.zeros(n * R, dtype=np.int64)
    out_off = 16 - pr if pr > 0 else 0
    in_off = ps
    last_off = ((ps + Rb - 1) >> 4) << 4
    most = Rb >> 4
    tiles = aligned_tiles(most, TILE * U) if most > 0 else 0
    for k in range(n):
        b0 = k * Rb - out_off
        vlo, vhi = (b0 + 15) >> 4, (b0 + Rb) >> 4
        covered = 0
        for j in range(tiles):
            start, lo, hi = aligned_tile(vlo, vhi, j, ref, TILE * U)
            if lo >= hi:
                continue
            off, ok = lanes(start, lo, hi, U)
            inb = in_off + lo * 16 - b0
            base, ph = inb & ~15, inb & 15
            rel = last_off - base
            hi_off = np.where(off + 16 < rel, off + 16, rel)
            for ld in (base + off, base + hi_off):
                assert ld.min() >= 0 and (ld + 16).max() <= last_off + 16, (n, e, R, ps, pr, U, k, j)
            o = lo + off[ok] // 16
            src = inb + off[ok]                       # input bytes of frame vector o: ps + 16*o - b0
            assert np.array_equal(src, ps + 16 * o - b0)
            assert src.min() >= ps and (src + 16).max() <= ps + Rb
            if ph:
                assert np.array_equal(hi_off[ok], off[ok] + 16), (n, e, R, ps, pr, U, k, j)
            for q in o:
                # frame byte 16*q is byte 16*q + out_off of the caller's output, element k*R + (16*q - b0)/e
                first = (16 * int(q) + out_off) // e
                assert first == k * R + (16 * int(q) - b0) // e and first + 16 // e <= n * R
                writes[first:first + 16 // e] += 1
                covered += 1
        assert covered == max(0, vhi - vlo), (n, e, R, ps, pr, U, k)   # the grid reaches every whole vector
        # the edge kernel: elements [0, head) and [tail, R) of the piece
        o0, o1 = vlo, vhi
        head, tail = (R, R) if o1 <= o0 else ((o0 * 16 - b0) // e, (o1 * 16 - b0) // e)
        writes[k * R:k * R + head] += 1
        writes[k * R + tail:k * R + R] += 1
    return writes


def _cases(rng, e):
    u = 16 // e
    lengths = [1, u - 1, u + 1, TILE * u - 1, TILE * u + 1, 2 * TILE * u + 3, 3 * TILE * u + u - 1,
               4 * TILE * u + 5]
    lengths += [rng.randrange(1, 6 * TILE * u) for _ in range(4)]
    return [R for R in lengths if R * e % 16]


@pytest.mark.parametrize("words", [False, True])
@pytest.mark.parametrize("e", [2, 4])
def test_phased_reduce_scatter_index_map(e, words):
    rng = random.Random(11 + e)
    phases = list(range(0, 16, e))
    for n in (1, 2, 3, 5, 8, 9, 17):
        for R in _cases(rng, e):
            for U in sorted({1, 2, 4, library_u(n)}):
                ps, pr = rng.choice(phases), rng.choice(phases)
                refs = [rng.randrange(0, 1 << 20) for _ in range(n)]
                w = emulate_rs(n, e, R, ps, pr, U, refs, words=words)
                assert (w == 1).all(), (n, e, R, ps, pr, U)


@pytest.mark.parametrize("e", [2, 4])
def test_phased_all_gather_index_map(e):
    rng = random.Random(21 + e)
    phases = list(range(0, 16, e))
    for n in (1, 2, 3, 5, 8, 9, 17):
        for R in _cases(rng, e):
            for U in sorted({1, 2, 4, library_u(n, "ag")}):
                ps, pr = rng.choice(phases), rng.choice(phases)
                w = emulate_ag(n, e, R, ps, pr, U, rng.randrange(0, 1 << 20))
                assert (w == 1).all(), (n, e, R, ps, pr, U)


@pytest.mark.parametrize("e", [2, 4])
def test_mixed_phase_reduce_scatter_words_index_map(e):
    """Reduce-scatter at mixed phases with 4-byte-aligned pointers: the phased kernel's word-aligned loads
    run on the callers' pointers with no frame shift (output vector o of slice c at byte 16*o, input at
    c*R*e + 16*o), the element-wise kernel takes elements [lanes*Rv, R) of every slice.  Every load is
    4-byte aligned and lies in the words holding the lane's input bytes, inside slice c (2-byte slices of
    an odd length take the next word as well); every output element is written once."""
    rng = random.Random(3 + e)
    u = 16 // e
    for n in (1, 2, 3, 8, 9, 17):
        for R in [1, 3, 4, 5, 63, 64 * u + 1] + [rng.randrange(1, 6 * TILE * u) for _ in range(4)]:
            Rb = R * e
            Rv = Rb // 16
            src = [4 * rng.randrange(0, 1 << 18) for _ in range(n)]       # 4-byte aligned, any 16-byte phase
            dst = [4 * rng.randrange(0, 1 << 18) for _ in range(n)]
            writes = np.zeros((n, R), dtype=np.int64)
            for c in range(n):
                for U in (1, 2):
                    if U != library_u(n):
                        continue
                    for j in range(aligned_tiles(Rv, TILE * U)):
                        start, lo, hi = aligned_tile(0, Rv, j, dst[c] >> 4, TILE * U)
                        if lo >= hi:
                            continue
                        off, ok = lanes(start, lo, hi, U)
                        a = c * Rb + lo * 16
                        whole = lo == start and hi == start + TILE * U
                        for r in range(n):
                            loads, nxt = rs_words_loads(src[r] + a, off, whole, U)
                            assert (loads % 4 == 0).all()
                            # inside the words that hold slice c's bytes
                            wlo, whi = (src[r] + c * Rb) & ~3, (src[r] + (c + 1) * Rb + 3) & ~3
                            assert loads.min() >= wlo and (loads + 16).max() <= whi, (n, R, c, r)
                            if nxt is not None:
                                assert e == 2 and (nxt + 4).max() <= whi, (n, R, c, r)
                            assert np.array_equal(loads[ok] + ((src[r] + a) & 3), src[r] + a + off[ok])
                        for q in lo + off[ok] // 16:
                            writes[c, u * q:u * q + u] += 1
            writes[:, u * Rv:] += 1
            assert (writes == 1).all(), (n, R)


@pytest.mark.parametrize("e", [2, 4])
def test_mixed_phase_all_gather_words_index_map(e):
    """All-gather at mixed phases with every pointer and the piece length whole 4-byte words: the phased
    kernel on the callers' pointers (output frame from byte 0, piece k at bytes [k*R*e, (k+1)*R*e)), one
    load per frame vector from its input bytes, every load 4-byte aligned and inside the piece; the
    element-wise kernel takes each piece's ends; every output element is written once."""
    rng = random.Random(7 + e)
    u = 16 // e
    for n in (1, 2, 3, 8, 9, 17):
        for R in [2, 4, 6, 64 * u + 2, 2 * TILE * u - 2] + [2 * rng.randrange(1, 3 * TILE * u) for _ in range(4)]:
            Rb = R * e
            assert Rb % 4 == 0
            src = [4 * rng.randrange(0, 1 << 18) for _ in range(n)]
            ref = 4 * rng.randrange(0, 1 << 18) >> 4
            U = library_u(n, "ag")
            writes = np.zeros(n * R, dtype=np.int64)
            most = Rb >> 4
            for k in range(n):
                b0 = k * Rb
                vlo, vhi = (b0 + 15) >> 4, (b0 + Rb) >> 4
                for j in range(aligned_tiles(most, TILE * U) if most > 0 else 0):
                    start, lo, hi = aligned_tile(vlo, vhi, j, ref, TILE * U)
                    if lo >= hi:
                        continue
                    off, ok = lanes(start, lo, hi, U)
                    inb = lo * 16 - b0
                    ld = src[k] + inb + off
                    assert (ld % 4 == 0).all()
                    assert ld.min() >= src[k] and (ld + 16).max() <= src[k] + Rb, (n, e, R, k, j)
                    for q in lo + off[ok] // 16:
                        writes[16 * q // e:16 * q // e + u] += 1
                head, tail = (R, R) if vhi <= vlo else ((vlo * 16 - b0) // e, (vhi * 16 - b0) // e)
                writes[k * R:k * R + head] += 1
                writes[k * R + tail:k * R + R] += 1
            assert (writes == 1).all(), (n, e, R)


@pytest.mark.parametrize("mistake", [{"slack": 16}, {"edge_shift": 1}, {"edge_shift": -1},
                                     {"words": True, "shift_mask": 15}])
def test_model_notices_planted_mistakes(mistake):
    """A clamp one block short, an edge range off by one element, or the word-aligned form shifting by
    the 16-byte phase instead of the word phase, fails the checks for some case."""
    rng = random.Random(5)
    failed = 0
    for n in (2, 3, 8):
        for R in _cases(rng, 4):
            try:
                w = emulate_rs(n, 4, R, 4, 0, 2, [0] * n, **mistake)
                failed += int(not (w == 1).all())
            except AssertionError:
                failed += 1
    assert failed > 0


def phased_rs_waves(n, e):
    """Wavefronts per workgroup of the library's phased reduce-scatter (4-byte types keep one at 16 ranks,
    up to 4 ranks eight)."""
    return 1 if (n == 16 and e == 4) else (8 if n <= 4 else 4)


@pytest.mark.parametrize("waves", [1, 2, 4, 8])
def test_multi_wave_workgroups_cover_every_tile_once(waves):
    """A workgroup of W wavefronts takes tiles j = blockIdx.x * W + wave; the grid has ceil(tiles / W)
    workgroups.  Every tile of the range is taken exactly once and the extra wavefronts of the last
    workgroup find an empty tile (their first vector lies past the range), so they write nothing."""
    rnd = random.Random(11 + waves)
    for _ in range(400):
        U = rnd.choice([1, 2])
        T = TILE * U
        length = rnd.randint(1, 40 * T)
        ref = rnd.randint(0, 4 * T)
        tiles = aligned_tiles(length, T)
        grid = (tiles + waves - 1) // waves
        covered = np.zeros(length, dtype=np.int64)
        for bx in range(grid):
            for w in range(waves):
                j = bx * waves + w
                start, lo, hi = aligned_tile(0, length, j, ref, T)
                if j >= tiles:
                    assert lo >= hi, (length, ref, T, j)
                if lo < hi:
                    covered[lo:hi] += 1
        assert (covered == 1).all()
    assert phased_rs_waves(8, 2) == 4 and phased_rs_waves(16, 4) == 1 and phased_rs_waves(16, 2) == 4
    assert phased_rs_waves(4, 4) == 8 and phased_rs_waves(2, 2) == 8
