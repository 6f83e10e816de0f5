"""Layout algebra beyond the hot path, on the host: logical_product,
coalesce, closed-form composition and the divide of nested modes.

The oracle's new definitions are pinned first -- the product by the closed
form of a concatenated colexicographic index, the nested divide by the flat
divide (itself pinned by the page's 1024 / 128 example), by a closed form of
the SM80 A-operand thread mode and by pointwise composition with the tiler.
Then the library's descriptors, evaluated with the oracle's crd2idx, must
give exactly the oracle's tables (composition: the pointwise A(B(c))).
"""
import random

import pytest

import tiled_layout_algebra_amd as tla
from oracle import layout as L

SM80_A = (((4, 8), (2, 2, 2)), ((32, 1), (16, 8, 128)))


def _table(desc):
    return L.Layout(*tla.layout_tuple(desc)).table()


def _leaves(desc):
    shape, stride = tla.layout_tuple(desc)
    return list(zip(L.flatten(shape), L.flatten(stride)))


def _random_layout(rng, max_modes=4, max_leaves=3, ext=(1, 5), strides=range(-3, 9),
                   max_size=2048):
    while True:
        shape, stride = [], []
        for _ in range(rng.randint(1, max_modes)):
            k = rng.randint(1, max_leaves)
            s = tuple(rng.randint(*ext) for _ in range(k))
            d = tuple(rng.choice(list(strides)) for _ in range(k))
            shape.append(s[0] if k == 1 else s)
            stride.append(d[0] if k == 1 else d)
        if L.size(tuple(shape)) <= max_size:
            return tuple(shape), tuple(stride)


# ------------------------------------------------------------ oracle pins

def test_oracle_product_is_concatenation_of_colex_indices():
    """out(i) = L(i mod |L|) + M(i div |L|): with L's modes first, the
    colexicographic index runs through L's coordinates fastest."""
    cases = [(((4, 8), (8, 1)), ((2,), (32,))), (SM80_A, ((3, 2), (1000, 7))),
             (((2, (3, 2)), (5, (1, 40))), ((4,), (-6,)))]
    for (ls, ld), (ms, md) in cases:
        a, b = L.Layout(ls, ld), L.Layout(ms, md)
        p = L.logical_product(a, b)
        assert p.size() == a.size() * b.size()
        assert p.table() == [a(i % a.size()) + b(i // a.size()) for i in range(p.size())]


def test_oracle_divide_modes_pins():
    # flat layouts: the same function as the pinned flat divide, by coordinate
    for shape, stride, tile in [((1024,), (1,), (128,)), ((12, 10), (10, 1), (4, 3)),
                                ((7, 9), (1, 7), (2, 4))]:
        lay = L.Layout(shape, stride)
        dm, dv = L.divide_modes(lay, tile), L.logical_divide(lay, tile)
        for i in range(dm.size()):
            c = L.idx2crd(i, dm.shape)
            pairs = tuple((c[2 * k], c[2 * k + 1]) for k in range(len(tile)))
            assert dm(i) == dv(pairs if len(pairs) > 1 else pairs[0])
    # the page's 1024 / 128 example: (e, t) -> 128 t + e
    dm = L.divide_modes(L.Layout((1024,), (1,)), (128,))
    assert dm.shape == (128, 8) and dm.table() == list(range(1024))
    # SM80 thread mode (4,8):(32,1) by 4: thread e + 4q owns 32e + q
    dm = L.divide_modes(L.Layout(*SM80_A), (4, 8))
    for i in range(dm.size()):
        e, q, v, _ = L.idx2crd(i, dm.shape)
        mode1 = L.Layout((2, 2, 2), (16, 8, 128))
        assert dm(i) == 32 * e + q + mode1(v)
    # a nested mode divided = the mode composed with (t, n/t):(1, t)
    for shape, stride, t in [(((4, 8),), ((32, 1),), 8), ((((2, 3), 4),), (((1, 2), 6),), 6)]:
        mode = L.Layout(shape[0], stride[0])
        n = mode.size()
        tiler = L.Layout((t, n // t), (1, t))
        assert L.divide_modes(L.Layout(shape, stride), (t,)).table() == \
            L.Composition(mode, tiler).table()


# --------------------------------------------------------- logical_product

def test_product_matches_oracle():
    rng = random.Random(11)
    for _ in range(200):
        a = _random_layout(rng, max_modes=3, max_leaves=2, max_size=128)
        b = _random_layout(rng, max_modes=3, max_leaves=2, max_size=32)
        if sum(len(L.flatten(x)) for x in (a[0], b[0])) > 16:
            continue
        got = tla.logical_product(tla.make_layout(*a), tla.make_layout(*b))
        want = L.logical_product(L.Layout(*a), L.Layout(*b))
        assert tla.layout_tuple(got) == (want.shape, want.stride)
        assert _table(got) == want.table()


def test_product_limits():
    big = tla.make_layout(tuple(range(2, 7)), (1,) * 5)
    with pytest.raises(tla.TlaError):
        tla.logical_product(big, big)  # 10 modes > 8


# ---------------------------------------------------------------- coalesce

def test_coalesce_keeps_the_function_and_cannot_merge_further():
    rng = random.Random(5)
    merged = 0
    for _ in range(400):
        shape, stride = _random_layout(rng)
        d = tla.make_layout(shape, stride)
        c = tla.coalesce(d)
        assert _table(c) == L.Layout(shape, stride).table()
        lv = _leaves(c)
        merged += len(lv) < len(L.flatten(shape))
        if L.size(shape) == 1:
            assert lv == [(1, 0)]
            continue
        assert all(s > 1 for s, _ in lv)
        for (s0, d0), (_, d1) in zip(lv, lv[1:]):
            assert d1 != s0 * d0
    assert merged > 100  # the random cases do exercise merging


def test_coalesce_examples():
    assert tla.layout_tuple(tla.coalesce(tla.make_layout(((2, 2), 4, 1), ((1, 2), 4, 7)))) == \
        ((16,), (1,))
    assert tla.layout_tuple(tla.coalesce(tla.make_layout((4, 8), (8, 1)))) == ((4, 8), (8, 1))
    assert tla.layout_tuple(tla.coalesce(tla.make_layout((1, 1), (5, 9)))) == ((1,), (0,))


# ----------------------------------------------------------- composition

def _admissible_b(rng, a_shape):
    """A B whose leaves walk whole runs of A's mixed radix: split A's extents
    into factors and pick a sub-range of the resulting radix points."""
    factors = []
    for s in a_shape:
        while s > 1:
            f = next(p for p in range(2, s + 1) if s % p == 0)
            factors.append(f)
            s //= f
    weights, w = [], 1
    for f in factors:
        weights.append(w)
        w *= f
    idx = list(range(len(factors)))
    rng.shuffle(idx)
    pick = sorted(idx[:rng.randint(1, len(idx))])
    # group consecutive picked factors into leaves, permute the leaves
    leaves, run = [], []
    for i in pick:
        if run and i != run[-1] + 1:
            leaves.append(run)
            run = []
        run.append(i)
    leaves.append(run)
    rng.shuffle(leaves)
    shape = tuple(L.size(tuple(factors[i] for i in r)) for r in leaves)
    stride = tuple(weights[r[0]] for r in leaves)
    return shape, stride


def test_composition_matches_pointwise():
    rng = random.Random(7)
    for _ in range(300):
        a_shape = tuple(rng.choice([2, 3, 4, 6, 8]) for _ in range(rng.randint(1, 3)))
        perm = list(range(len(a_shape)))
        rng.shuffle(perm)
        a_stride, acc = [0] * len(a_shape), 1
        for k in perm:
            a_stride[k] = acc
            acc *= a_shape[k]
        a_stride = tuple(a_stride)
        b_shape, b_stride = _admissible_b(rng, a_shape)
        A, B = tla.make_layout(a_shape, a_stride), tla.make_layout(b_shape, b_stride)
        R = tla.composition(A, B)  # admissible by construction: must succeed
        want = L.Composition(L.Layout(a_shape, a_stride), L.Layout(b_shape, b_stride)).table()
        assert _table(R) == want
        assert R.n_modes == B.n_modes


def test_composition_random_pairs():
    """Arbitrary pairs: whenever a closed form is returned it is exact, and
    the pairs it refuses include ones with no single-leaf form."""
    rng = random.Random(3)
    ok = refused = 0
    for _ in range(600):
        a_shape = tuple(rng.randint(1, 6) for _ in range(rng.randint(1, 3)))
        a_stride = tuple(rng.randint(0, 9) for _ in a_shape)
        size_a = L.size(a_shape)
        b_shape = tuple(rng.randint(1, 4) for _ in range(rng.randint(1, 3)))
        b_stride = tuple(rng.randint(0, 6) for _ in b_shape)
        b = L.Layout(b_shape, b_stride)
        if max(b.table()) >= size_a:
            with pytest.raises(tla.TlaError) as e:
                tla.composition(tla.make_layout(a_shape, a_stride), tla.make_layout(b_shape, b_stride))
            assert e.value.status == tla.ERR_INVALID_ARG
            continue
        try:
            R = tla.composition(tla.make_layout(a_shape, a_stride), tla.make_layout(b_shape, b_stride))
        except tla.TlaError as e:
            assert e.status == tla.ERR_UNSUPPORTED
            refused += 1
            continue
        ok += 1
        assert _table(R) == L.Composition(L.Layout(a_shape, a_stride), b).table()
    assert ok > 150 and refused > 20


def test_composition_examples():
    # a 2x2 column-major view of the 4x8 row-major tile
    R = tla.composition(tla.make_layout((4, 8), (8, 1)), tla.make_layout((2, 2), (1, 4)))
    assert tla.layout_tuple(R) == ((2, 2), (8, 1))
    # indices 0, 2, 4 of a 4x8 row-major tile land on (0,0), (2,0), (0,1):
    # values 0, 16, 1 -- no single stride, so no closed form
    with pytest.raises(tla.TlaError) as e:
        tla.composition(tla.make_layout((4, 8), (8, 1)), tla.make_layout(3, 2))
    assert e.value.status == tla.ERR_UNSUPPORTED
    # the pages' chain: a vector, arranged into a matrix, matrices batched.
    # memory: 2 matrices of 6x8 row-major; a matrix view (8,6) column by
    # column; vectors of 2 along that view's columns
    mem = tla.make_layout((8, 6, 2), (1, 8, 48))
    mat = tla.make_layout(((2, 4), 6, 2), ((1, 2), 8, 48))
    vec = tla.make_layout((2, 48), (1, 2))
    step1 = tla.composition(mem, mat)
    step2 = tla.composition(step1, vec)
    want = L.Composition(L.Composition(L.Layout((8, 6, 2), (1, 8, 48)),
                                       L.Layout(((2, 4), 6, 2), ((1, 2), 8, 48))),
                         L.Layout((2, 48), (1, 2))).table()
    assert _table(step2) == want
    # associativity: (A o B) o C == A o (B o C) pointwise
    other = tla.composition(mem, tla.composition(mat, vec))
    assert _table(other) == want


# ----------------------------------------------------- divide of nested modes

@pytest.mark.parametrize("shape,stride,tile", [
    (SM80_A[0], SM80_A[1], (4, 2)),
    (SM80_A[0], SM80_A[1], (8, 4)),
    (SM80_A[0], SM80_A[1], (32, 8)),
    ((((4, 8), 2)), (((2, 8), 1)), (8, 2)),          # ldmatrix .x1 lanes
    (((2, 3), 4), ((1, 2), 6), (3, 2)),
    ((1024,), (1,), (128,)),                           # the page's example
    ((12, 10), (10, 1), (5, 3)),                       # ragged flat modes
])
def test_divide_modes_matches_oracle(shape, stride, tile):
    d = tla.logical_divide_modes(tla.make_layout(shape, stride), tile)
    want = L.divide_modes(L.Layout(shape, stride), tile)
    s, _ = tla.layout_tuple(d)
    assert tuple(L.size(m) for m in s) == want.shape
    assert _table(d) == want.table()


def test_divide_modes_refusals():
    with pytest.raises(tla.TlaError) as e:   # nested mode, tile does not divide
        tla.logical_divide_modes(tla.make_layout(SM80_A[0], SM80_A[1]), (5, 2))
    assert e.value.status == tla.ERR_UNSUPPORTED
    with pytest.raises(tla.TlaError):         # 5 modes -> 10 > 8
        tla.logical_divide_modes(tla.make_layout((2,) * 5, (1,) * 5), (1,) * 5)


def test_divide_modes_random_nested():
    rng = random.Random(9)
    checked = 0
    for _ in range(300):
        shape, stride = _random_layout(rng, max_modes=3, max_leaves=3, ext=(1, 4),
                                       strides=range(0, 7))
        tile = []
        for s in shape:
            n = L.size(s)
            divs = [t for t in range(1, n + 1) if n % t == 0]
            tile.append(rng.choice(divs) if not L.is_int(s) else rng.randint(1, n + 1))
        d = tla.make_layout(shape, stride)
        want = L.divide_modes(L.Layout(shape, stride), tuple(tile))
        try:
            got = tla.logical_divide_modes(d, tile)
        except tla.TlaError as e:
            assert e.status == tla.ERR_UNSUPPORTED
            continue
        checked += 1
        assert _table(got) == want.table()
    assert checked > 150
