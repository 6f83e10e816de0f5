"""Pins of the scalar layout oracle against what the pages fix: printed
examples and tables (tests/golden/), closed forms, invariants and brute
force on tiny cases.  CPU only."""
import itertools
import random

import pytest

from oracle import layout as L
from tests.golden_io import keyed, records


# ------------------------------------------------ crd2idx / idx2crd (P1)

def test_row_major_4x8_page_example():
    g = keyed("layout_4x8_row_major.txt")
    shape = tuple(int(x) for x in g["shape"])
    stride = tuple(int(x) for x in g["stride"])
    lay = L.Layout(shape, stride)
    rs, cs = int(g["row_step"][0]), int(g["col_step"][0])
    # stepping one row / one column moves by the printed amounts
    for i in range(shape[0]):
        for j in range(shape[1]):
            if i + 1 < shape[0]:
                assert lay(i + 1, j) - lay(i, j) == rs
            if j + 1 < shape[1]:
                assert lay(i, j + 1) - lay(i, j) == cs
    assert lay(0, 0) == 0
    # row-major 4x8 is a bijection onto 0..31 ("a bijective function")
    assert sorted(lay(i, j) for i in range(4) for j in range(8)) == list(range(32))
    # the generator for row-major strides reproduces the printed stride
    assert L.row_major(shape).stride == stride
    # colexicographic 1-D walk: first mode fastest
    assert lay.table()[:8] == [0, 8, 16, 24, 1, 9, 17, 25]


def test_idx2crd_colexicographic_and_inverse():
    for shape in [(4, 8), (3, 5, 2), ((4, 8), (2, 2, 2)), ((2, 3), 5, (1, 4))]:
        n = L.size(shape)
        seen = set()
        for i in range(n):
            c = L.idx2crd(i, shape)
            # the colexicographic (column-major) layout of the shape inverts it
            cm = _colex_layout(shape)
            assert L.crd2idx(c, shape, cm) == i
            seen.add(repr(c))
        assert len(seen) == n
    with pytest.raises(IndexError):
        L.idx2crd(32, (4, 8))


def _colex_layout(shape):
    """Strides of the compact colexicographic layout of a nested shape."""
    acc = [1]

    def walk(s):
        if L.is_int(s):
            d = acc[0]
            acc[0] *= s
            return d
        return tuple(walk(x) for x in s)
    return walk(shape)


def test_crd2idx_is_dot_product_brute_force():
    rnd = random.Random(7)
    for _ in range(200):
        r = rnd.randint(1, 4)
        shape = tuple(rnd.randint(1, 5) for _ in range(r))
        stride = tuple(rnd.randint(-6, 40) for _ in range(r))
        lay = L.Layout(shape, stride)
        for crd in itertools.product(*[range(s) for s in shape]):
            assert lay(*crd) == sum(c * d for c, d in zip(crd, stride))


def test_integer_coordinate_into_nested_mode():
    # an integer for a nested mode is that mode's colexicographic index
    shape, stride = ((4, 8), 3), ((32, 1), 1000)
    assert L.crd2idx((5, 2), shape, stride) == (5 % 4) * 32 + (5 // 4) * 1 + 2 * 1000


# --------------------------------------------- printed operand tables (P4-P6)

def test_ldmatrix_x1_printed_table():
    for rec in records("ldmatrix_x1.txt"):
        lane, r0, c0, r1, c1 = (int(x) for x in rec)
        assert L.ldmatrix_x1(lane) == [(r0, c0), (r1, c1)]
    # the 32 lanes cover the 8x8 matrix exactly once
    cover = [rc for lane in range(32) for rc in L.ldmatrix_x1(lane)]
    assert sorted(cover) == [(r, c) for r in range(8) for c in range(8)]


def test_ldmatrix_x1_as_hierarchical_layout():
    # lane -> (row, col) as a TV layout ((4,8),2):((2,8),1) into row*8+col
    tv = L.Layout(((4, 8), 2), ((2, 8), 1))
    for lane in range(32):
        for h in range(2):
            idx = tv((lane, h))
            assert (idx // 8, idx % 8) == L.ldmatrix_x1(lane)[h]


def test_ldmatrix_x4_printed_table_and_example():
    mats = [[int(x) for x in r[1:]] for r in records("ldmatrix_x4.txt") if r[0] == "mat"]
    assert len(mats) == 4
    for mat, tlo, thi, mlo, mhi, klo, khi, reg in mats:
        # register `reg` of every thread holds an element of sub-matrix `mat`
        for t in range(32):
            for h in range(2):
                m, k = L.ldmatrix_x4(t)[2 * reg + h]
                assert mlo <= m <= mhi and klo <= k <= khi
        assert thi - tlo == 7  # eight lanes give the eight row addresses
    for r in records("ldmatrix_x4.txt"):
        if r[0] != "example":
            continue
        t, reg, row, clo, chi = (int(x) for x in r[1:])
        assert L.ldmatrix_x4(t)[2 * reg] == (row, clo)
        assert L.ldmatrix_x4(t)[2 * reg + 1] == (row, chi)
    cover = [rc for t in range(32) for rc in L.ldmatrix_x4(t)]
    assert sorted(cover) == [(m, k) for m in range(16) for k in range(16)]


def test_sm80_a_layout_matches_x4_table_and_thread0():
    g = keyed("sm80_a_layout.txt")
    assert L.SM80_A_LAYOUT.shape == ((4, 8), (2, 2, 2))
    assert L.SM80_A_LAYOUT.stride == ((32, 1), (16, 8, 128))
    # every (t, v) agrees with the ldmatrix .x4 register order (v = h + 2j)
    for t in range(32):
        assert [L.sm80_a_coord(t, v) for v in range(8)] == L.ldmatrix_x4(t)
    vals = [int(x) for x in g["thread0"]]
    assert [L.sm80_a_coord(0, v) for v in range(8)] == list(zip(vals[0::2], vals[1::2]))
    # each mode's stride moves along the axis the page's mode table names
    for rec in records("sm80_a_layout.txt"):
        if rec[0] != "mode":
            continue
        _, name, ext, stride, axis, step = rec
        idx = int(stride)
        assert (idx % 16, idx // 16) == ((int(step), 0) if axis == "m" else (0, int(step)))


# ------------------------------------------------------ divides (P2, Q1, Q6)

def test_logical_divide_1024_by_128():
    g = keyed("logical_divide_1024_by_128.txt")
    n, t = int(g["extent"][0]), int(g["tile"][0])
    d = L.logical_divide(L.Layout(n, 1), t)
    assert sorted(d.shape[0]) == sorted([int(g["num_tiles"][0]), int(g["tile_size"][0])])
    assert d.shape == ((128, 8),)  # (inside-tile, tile-index) reading
    for tile in range(8):
        for e in range(128):
            assert d(((e, tile),)) == 128 * tile + e
    assert L.size(d.shape) == 1024


def test_logical_divide_is_composition_with_tiler():
    # dividing n:s by t is the composition of n:s with (t, n/t):(1, t)
    rnd = random.Random(3)
    for _ in range(50):
        t = rnd.randint(1, 9)
        n = t * rnd.randint(1, 9)
        s = rnd.randint(1, 5)
        base = L.Layout(n, s)
        comp = L.Composition(base, L.Layout((t, n // t), (1, t)))
        d = L.logical_divide(base, t)
        for i in range(n):
            assert d(L.idx2crd(i, d.shape)) == comp(i)


def test_logical_divide_ragged_in_range():
    d = L.logical_divide(L.Layout((10, 7), (7, 1)), (4, 3))
    assert d.shape == ((4, 3), (3, 3))
    inside = set()
    for i in range(d.size()):
        c = L.idx2crd(i, d.shape)
        oc = d.original_coord(c)
        assert d.in_range(c) == (oc[0] < 10 and oc[1] < 7)
        if d.in_range(c):
            inside.add(oc)
            assert d(c) == oc[0] * 7 + oc[1]
    assert len(inside) == 70


def test_tiled_divide_and_block_slice():
    # the transpose kernel's tiling: 32x32 blocks of an M x N row-major tensor
    M, N = 96, 64
    S = L.row_major((M, N))
    td = L.tiled_divide(S, (32, 32))
    assert td.shape == ((32, 32), 3, 2)
    for bx in range(3):
        for by in range(2):
            tile = td.tile_at(bx, by)
            for e0 in range(0, 32, 7):
                for e1 in range(0, 32, 5):
                    assert tile(e0, e1) == (32 * bx + e0) * N + (32 * by + e1)


# ------------------------------------------------------- local_partition (Q8)

def test_local_partition_transpose_kernel():
    thr = L.row_major((8, 32))
    owned_all = []
    for tid in range(256):
        own = L.local_partition(lambda r, c: (r, c), (32, 32), thr, tid)
        assert len(own) == 4
        r0, c0 = tid // 32, tid % 32
        assert own == [(r0 + 8 * i, c0) for i in range(4)]
        owned_all += own
    assert sorted(owned_all) == [(r, c) for r in range(32) for c in range(32)]


def test_transpose_by_layouts_equals_definition():
    # the page's transpose: copy each thread's partition of a row-major
    # tile into the column-major view of the same tile
    M, N = 64, 96
    src = list(range(M * N))
    dst = [None] * (M * N)
    S, DT = L.row_major((M, N)), L.col_major((M, N))
    tS, tD = L.tiled_divide(S, (32, 32)), L.tiled_divide(DT, (32, 32))
    thr = L.row_major((8, 32))
    for bx in range(M // 32):
        for by in range(N // 32):
            fs, fd = tS.tile_at(bx, by), tD.tile_at(bx, by)
            for tid in range(256):
                for a, b in zip(L.local_partition(fs, (32, 32), thr, tid),
                                L.local_partition(fd, (32, 32), thr, tid)):
                    dst[b] = src[a]
    for m in range(M):
        for n in range(N):
            assert dst[m + n * M] == src[m * N + n]


# --------------------------------------------------- thread map (P3, P7, P8)

def test_thread_map_page_example():
    g = keyed("thread_map_64x64_t128_v4_i8.txt")
    R, C, T, V, I = (int(g[k][0]) for k in "R C T V I".split())
    tm = L.StripMinedThreadMap(R, C, T, V, I)
    assert R * C == T * V * I == int(g["elements"][0])
    assert tm.G == int(g["column_groups"][0])
    assert tm.S == int(g["row_stride"][0])
    for rec in records("thread_map_64x64_t128_v4_i8.txt"):
        if rec[0] != "thread":
            continue
        t = int(rec[1])
        group, anchor = int(rec[3]), int(rec[5])
        assert t % tm.G == group and t // tm.G == anchor
        ci = rec.index("cols")
        ri = rec.index("rows") if "rows" in rec else len(rec)
        cols = [int(x) for x in rec[ci + 1:ri]]
        assert [tm.coord(t, 0, v)[1] for v in range(V)] == cols
        if "rows" in rec:
            rows = [int(x) for x in rec[ri + 1:]]
            assert [tm.coord(t, it, 0)[0] for it in range(I)] == rows


def test_thread_map_wave_rows():
    # The page's own formula puts threads 32-47 on row 2 and 48-63 on row 3
    # at iteration 0 (the prose says row 3 for all of 32-63; the formula
    # wins).  A 64-wide wavefront (threads 0-63) covers rows 0-3, cols 0-63.
    tm = L.StripMinedThreadMap(64, 64, 128, 4, 8)
    assert {tm.coord(t, 0, 0)[0] for t in range(32, 48)} == {2}
    assert {tm.coord(t, 0, 0)[0] for t in range(48, 64)} == {3}
    cells = {tm.coord(t, 0, v) for t in range(64) for v in range(4)}
    assert cells == {(r, c) for r in range(4) for c in range(64)}


def test_thread_map_tv_layout_equals_formula():
    tm = L.StripMinedThreadMap(64, 64, 128, 4, 8)
    tv = tm.tv_layout()
    assert tv.shape == ((16, 8), (4, 8)) and tv.stride == ((4, 64), (1, 512))
    assert tv((50, 0)) == 3 * 64 + 8
    for t in range(128):
        for it in range(8):
            for v in range(4):
                assert tv((t, v + 4 * it)) == tm.index(t, it, v)
    assert tm.table() == [tv(i) for i in range(4096)]


def test_thread_map_tile_equation_enforced():
    with pytest.raises(ValueError):
        L.StripMinedThreadMap(64, 64, 128, 4, 4)  # 64*64 != 128*4*4
    with pytest.raises(ValueError):
        L.StripMinedThreadMap(64, 60, 120, 8, 4)  # 8 does not divide 60


def _all_maps(limit_rc=32, limit_t=128):
    for R in [1, 2, 3, 4, 8, 16, 32]:
        for C in [1, 2, 4, 8, 12, 16, 32]:
            if R > limit_rc or C > limit_rc:
                continue
            for V in [1, 2, 4, 8]:
                if C % V:
                    continue
                G = C // V
                for I in [1, 2, 4, 8]:
                    if R % I:
                        continue
                    T = R * C // (V * I)
                    if T == 0 or T > limit_t or T % G or (R // I) != T // G:
                        continue
                    yield R, C, T, V, I


def test_thread_map_bijection_and_predicate_brute_force():
    n_maps = 0
    for R, C, T, V, I in _all_maps():
        for contig in (1, 0):
            if contig == 0:
                # column-contiguous variant: swap roles, keep the equation
                if R % V or C % I or T % (R // V) or (C // I) != T // (R // V):
                    continue
            tm = L.StripMinedThreadMap(R, C, T, V, I, contig)
            n_maps += 1
            cells = [tm.coord(t, it, v) for t in range(T) for it in range(I) for v in range(V)]
            assert sorted(cells) == [(r, c) for r in range(R) for c in range(C)]
            idx = tm.table()
            assert sorted(idx) == list(range(R * C))
            # every residue: the mask keeps exactly the in-range elements
            for M in range(R + 1):
                for N in range(C + 1):
                    kept = {tm.coord(t, it, v) for t in range(T) for it in range(I)
                            for v in range(V) if tm.valid(t, it, v, M, N)}
                    assert kept == {(r, c) for r in range(M) for c in range(N)}
    assert n_maps > 30


def test_thread_map_predicate_m63():
    g = keyed("thread_map_predicate_m63.txt")
    tm = L.StripMinedThreadMap(*(int(g[k][0]) for k in "R C T V I".split()))
    M, N = int(g["M"][0]), int(g["N"][0])
    t_lo, t_hi = (int(x) for x in g["masked_threads"])
    it_m, row_m = int(g["masked_iteration"][0]), int(g["masked_row"][0])
    masked = {(t, it) for t in range(128) for it in range(8)
              if not all(tm.valid(t, it, v, M, N) for v in range(4))}
    assert masked == {(t, it_m) for t in range(t_lo, t_hi + 1)}
    assert all(tm.coord(t, it, 0)[0] == row_m for t, it in masked)
    # the page's vector-granularity form agrees when V divides N
    for t in range(128):
        for it in range(8):
            assert tm.valid_page_form(t, it, M, N) == all(tm.valid(t, it, v, M, N) for v in range(4))


# ---------------------------------------------------- composition (Q4)

def test_composition_pointwise():
    A = L.Layout((4, 8), (8, 1))         # row-major 4x8
    B = L.Layout((8, 4), (4, 1))         # walk it as an 8x4 row-major view
    comp = L.Composition(A, B)
    for i in range(32):
        # B(i) is a 1-D index into A's colexicographic domain
        b = B(i)
        r, c = b % 4, b // 4
        assert comp(i) == 8 * r + c
    with pytest.raises(IndexError):
        L.Composition(L.Layout(4, 1), L.Layout(8, 1))(5)


def test_composition_with_identity_is_identity():
    rnd = random.Random(11)
    for _ in range(30):
        shape = tuple(rnd.randint(1, 4) for _ in range(3))
        stride = tuple(rnd.randint(0, 9) for _ in range(3))
        A = L.Layout(shape, stride)
        ident = L.Layout(L.size(shape), 1)
        comp = L.Composition(A, ident)
        assert comp.table() == A.table()


def test_xor_swizzle_rows_hit_distinct_chunks():
    # the 8 rows one ldmatrix reads, same logical 16-byte chunk, land in 8
    # different physical chunks; per row the swizzle is a permutation
    for chunk in range(8):
        assert sorted(L.xor_swizzle_chunk(r, chunk) for r in range(8)) == list(range(8))
    for r in range(64):
        assert sorted(L.xor_swizzle_chunk(r, c) for c in range(8)) == list(range(8))
