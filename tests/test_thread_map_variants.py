"""Thread-map variants of the strip-mined map walk-through as options: the
threads-per-row override (section 2.2) and the swizzled map (section 5.3),
beside the column-major variant (section 3.4) the hot path already uses.

Oracle pins: with the options at their defaults the map is the page's
(whose worked example is pinned elsewhere); every well-formed variant is a
bijection onto the tile with an exact predicate (brute force); threads of
one row cover one contiguous run per pass; the swizzle permutes the column
groups of each row and, with the GEMM slab's parameters, spreads the rows
a quarter-wave reads over 16 distinct 16-byte LDS bank groups.  Then the
library's TV-layout descriptors must match the oracle's (the device
evaluation is in the GPU layout tests)."""
import itertools

import pytest

import tiled_layout_algebra_amd as tla
from oracle import layout as L


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


def _variants(max_rc=16, threads=(1, 2, 4, 8, 16, 32, 64)):
    """Every well-formed (R, C, T, V, I, contig, G) with R, C <= max_rc."""
    for R, C in itertools.product(range(1, max_rc + 1), repeat=2):
        for T in threads:
            if (R * C) % T:
                continue
            for V in _divisors(R * C // T):
                I = R * C // (T * V)
                for contig in (0, 1):
                    Q = C if contig else R
                    if Q % V:
                        continue
                    for G in _divisors(Q // V):
                        try:
                            m = L.StripMinedThreadMap(R, C, T, V, I, contig, threads_per_row=G)
                        except ValueError:
                            continue
                        yield m


def test_defaults_are_the_page_map():
    for R, C, T, V, I in [(64, 64, 128, 4, 8), (16, 8, 32, 2, 2), (8, 32, 16, 4, 4)]:
        base = L.StripMinedThreadMap(R, C, T, V, I)
        explicit = L.StripMinedThreadMap(R, C, T, V, I, 1, threads_per_row=C // V,
                                         swizzle_shift=-1)
        assert explicit.table() == base.table()
    # the page's worked example, thread 50: columns 8-11, rows 3, 11, ..., 59
    m = L.StripMinedThreadMap(64, 64, 128, 4, 8, 1, threads_per_row=16)
    assert [m.coord(50, it, 0) for it in range(8)] == [(3 + 8 * it, 8) for it in range(8)]


def test_every_variant_is_a_bijection_with_an_exact_predicate():
    n = 0
    for m in _variants():
        seen = sorted(m.index(t, it, v) for t in range(m.T) for it in range(m.I)
                      for v in range(m.V))
        assert seen == list(range(m.R * m.C)), (m.R, m.C, m.T, m.V, m.I, m.contig, m.G)
        for Mr, Nr in [(m.R - 1, m.C), (m.R, m.C - 1), (m.R // 2, m.C // 2)]:
            kept = sum(m.valid(t, it, v, Mr, Nr) for t in range(m.T) for it in range(m.I)
                       for v in range(m.V))
            assert kept == max(Mr, 0) * max(Nr, 0)
        n += 1
    assert n > 500


def test_threads_of_a_row_cover_one_contiguous_run_per_pass():
    for m in _variants(max_rc=12):
        if m.contig != 1:
            continue
        for it in range(m.I):
            for r0 in range(0, m.T, m.G):
                cols = sorted(m.coord(t, it, v)[1] for t in range(r0, r0 + m.G)
                              for v in range(m.V))
                rows = {m.coord(t, it, 0)[0] for t in range(r0, r0 + m.G)}
                assert len(rows) == 1
                start = cols[0]
                assert cols == list(range(start, start + m.G * m.V))
                assert start % (m.G * m.V) == 0


def test_swizzle_permutes_each_row():
    for R, C, T, V, I, G, s in [(16, 64, 64, 4, 4, 16, 0), (32, 128, 128, 8, 4, 16, 1),
                                (64, 8, 64, 1, 8, 8, 1), (16, 32, 32, 2, 8, 8, 2),
                                (8, 64, 16, 4, 8, 4, 0)]:
        plain = L.StripMinedThreadMap(R, C, T, V, I, 1, threads_per_row=G)
        swz = L.StripMinedThreadMap(R, C, T, V, I, 1, threads_per_row=G, swizzle_shift=s)
        groups = C // V
        for t in range(T):
            for it in range(I):
                r, c = plain.coord(t, it, 0)
                r2, c2 = swz.coord(t, it, 0)
                assert r2 == r
                assert c2 // V == (c // V) ^ ((r >> s) % groups)
                if r < (1 << s):
                    assert c2 == c
        seen = sorted(swz.index(t, it, v) for t in range(T) for it in range(I) for v in range(V))
        assert seen == list(range(R * C))


def test_swizzle_spreads_lds_banks_for_the_gemm_slab():
    """A 256-row slab of 128-byte rows (8 chunks of 16 bytes), one chunk per
    access (V = 1), 256 threads, swizzle shift 1.  Thread t at iteration it
    writes the lane-linear LDS slot the unswizzled map gives it and fetches
    the global chunk the swizzled map gives it.  The 16 rows a quarter-wave
    reads at one logical chunk then sit in 16 distinct 16-byte groups of a
    256-byte bank window (64 banks x 4 bytes); unswizzled, in two."""
    swz = L.StripMinedThreadMap(256, 8, 256, 1, 8, 1, swizzle_shift=1)
    plain = L.StripMinedThreadMap(256, 8, 256, 1, 8, 1)
    where = {}
    for t in range(256):
        for it in range(8):
            where[swz.coord(t, it, 0)] = plain.index(t, it, 0) * 16  # LDS byte address
    assert len(where) == 256 * 8
    for base in range(0, 256, 16):
        for c in range(8):
            groups = {(where[(base + r, c)] // 16) % 16 for r in range(16)}
            assert len(groups) == 16
            assert len({((base + r) * 8 + c) % 16 for r in range(16)}) == 2


@pytest.mark.parametrize("R,C,T,V,I,contig,G", [
    (64, 64, 128, 4, 8, 1, 16), (64, 64, 128, 4, 8, 1, 8), (64, 64, 128, 4, 8, 1, 4),
    (64, 64, 128, 4, 8, 0, 8), (32, 128, 64, 8, 8, 1, 4), (16, 16, 16, 2, 8, 1, 2),
])
def test_descriptor_matches_oracle(R, C, T, V, I, contig, G):
    d = tla.thread_map_ex(R, C, T, V, I, contig, G)
    m = L.StripMinedThreadMap(R, C, T, V, I, contig, threads_per_row=G)
    tv = m.tv_layout()
    assert tla.layout_tuple(d) == (tv.shape, tv.stride)
    assert L.Layout(*tla.layout_tuple(d)).table() == m.table()


def test_descriptor_refusals():
    with pytest.raises(tla.TlaError):
        tla.thread_map_ex(64, 64, 128, 4, 8, 1, 3)     # 3 does not divide 16 groups
    with pytest.raises(tla.TlaError):
        tla.thread_map_ex(64, 64, 128, 4, 8, 1, 32)    # 32 > 16 groups
    with pytest.raises(tla.TlaError):
        tla.thread_map_ex(64, 64, 128, 4, 8, 1, -2)    # negative override
    with pytest.raises(tla.TlaError):
        tla.thread_map_ex(64, 64, 96, 4, 8, 1, 16)     # tile equation fails
