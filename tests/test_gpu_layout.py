"""Device layout module parity: tla_layout_eval and tla_thread_map_eval
against the scalar layout oracle, value for value -- the pages' layouts,
the divide and thread-map descriptors, random flat and nested layouts,
pointwise compositions, and the thread map's predicate masks."""
import random

import numpy as np
import pytest
import torch

import tiled_layout_algebra_amd as tla
from oracle import layout as L
from tests.test_oracle_layout import _all_maps

pytestmark = pytest.mark.gpu


def _dev_table(outer, inner=None):
    n = tla.layout_size(inner if inner is not None else outer)
    out = torch.full((max(n, 1),), -7, dtype=torch.int64, device="cuda")
    tla.layout_eval(outer, inner, out, n)
    torch.cuda.synchronize()
    return out[:n].cpu().tolist()


def _oracle_layout(desc):
    return L.Layout(*tla.layout_tuple(desc))


PAGE_LAYOUTS = [
    ((4, 8), (8, 1)),                                   # 4x8 row-major
    (((4, 8), (2, 2, 2)), ((32, 1), (16, 8, 128))),     # SM80 A operand
    (((4, 8), 2), ((2, 8), 1)),                         # ldmatrix .x1 lanes
    ((1024,), (1,)),
]


@pytest.mark.parametrize("shape,stride", PAGE_LAYOUTS)
def test_page_layouts(shape, stride):
    d = tla.make_layout(shape, stride)
    assert _dev_table(d) == L.Layout(shape, stride).table()


def test_thread_map_descriptor_on_device():
    d = tla.thread_map(64, 64, 128, 4, 8)
    tm = L.StripMinedThreadMap(64, 64, 128, 4, 8)
    assert _dev_table(d) == tm.table()


@pytest.mark.parametrize("shape,stride,tile", [((1024,), (1,), (128,)), ((96, 64), (64, 1), (32, 32)),
                                               ((10, 7), (7, 1), (4, 3))])
def test_divides_on_device(shape, stride, tile):
    base = tla.make_layout(shape, stride)
    for desc, ref in [(tla.logical_divide(base, tile), L.logical_divide(L.Layout(shape, stride), tile)),
                      (tla.tiled_divide(base, tile), L.tiled_divide(L.Layout(shape, stride), tile))]:
        got = _dev_table(desc)
        assert got == [ref(L.idx2crd(i, ref.shape)) for i in range(ref.size())]


def _random_layout(rnd):
    n_modes = rnd.randint(1, 4)
    shape, stride = [], []
    for _ in range(n_modes):
        if rnd.random() < 0.4:
            k = rnd.randint(2, 3)
            shape.append(tuple(rnd.randint(1, 5) for _ in range(k)))
            stride.append(tuple(rnd.randint(-20, 200) for _ in range(k)))
        else:
            shape.append(rnd.randint(1, 9))
            stride.append(rnd.randint(-20, 200))
    return tuple(shape), tuple(stride)


def test_random_layouts():
    rnd = random.Random(1234)
    for _ in range(60):
        shape, stride = _random_layout(rnd)
        d = tla.make_layout(shape, stride)
        assert _dev_table(d) == L.Layout(shape, stride).table(), (shape, stride)


def test_compositions():
    A = tla.make_layout((4, 8), (8, 1))
    B = tla.make_layout((8, 4), (4, 1))
    ref = L.Composition(L.Layout((4, 8), (8, 1)), L.Layout((8, 4), (4, 1)))
    assert _dev_table(A, B) == ref.table()
    rnd = random.Random(99)
    done = 0
    while done < 40:
        oshape, ostride = _random_layout(rnd)
        osz = L.size(oshape)
        ishape = tuple(rnd.randint(1, 6) for _ in range(rnd.randint(1, 3)))
        istride = tuple(rnd.randint(0, max(1, osz // 4)) for _ in ishape)
        inner = L.Layout(ishape, istride)
        if max(inner.table()) >= osz:
            continue
        got = _dev_table(tla.make_layout(oshape, ostride), tla.make_layout(ishape, istride))
        assert got == L.Composition(L.Layout(oshape, ostride), inner).table()
        done += 1


def _map_eval(R, C, T, V, I, contig, rows, cols):
    n = T * V * I
    idx = torch.full((n,), -1, dtype=torch.int64, device="cuda")
    val = torch.full((n,), 9, dtype=torch.uint8, device="cuda")
    tla.thread_map_eval(R, C, T, V, I, contig, rows, cols, idx, val)
    torch.cuda.synchronize()
    return idx.cpu().tolist(), val.cpu().tolist()


def test_thread_map_eval_page_example_and_predicate():
    tm = L.StripMinedThreadMap(64, 64, 128, 4, 8)
    idx, val = _map_eval(64, 64, 128, 4, 8, 1, 63, 64)
    assert idx == tm.table()
    for t in range(128):
        for it in range(8):
            for v in range(4):
                i = t + 128 * (v + 4 * it)
                assert val[i] == int(tm.valid(t, it, v, 63, 64))
    assert [idx[50 + 128 * 4 * it] for it in range(8)] == [r * 64 + 8 for r in (3, 11, 19, 27, 35, 43, 51, 59)]


def test_thread_map_eval_brute_force():
    rnd = random.Random(5)
    for R, C, T, V, I in _all_maps():
        for contig in (1, 0):
            try:
                tm = L.StripMinedThreadMap(R, C, T, V, I, contig)
            except ValueError:
                continue
            rows, cols = rnd.randint(0, R), rnd.randint(0, C)
            idx, val = _map_eval(R, C, T, V, I, contig, rows, cols)
            assert idx == tm.table()
            want = [0] * (T * V * I)
            for it in range(I):
                for v in range(V):
                    for t in range(T):
                        want[t + T * (v + V * it)] = int(tm.valid(t, it, v, rows, cols))
            assert val == want


# -------------------------------------------- layout algebra results on device

def test_algebra_results_on_device():
    """Closed-form composition, nested divide, product and coalesce
    descriptors evaluated by the device module, against the oracle's
    pointwise definitions."""
    sm80 = (((4, 8), (2, 2, 2)), ((32, 1), (16, 8, 128)))
    # the pages' chain: vectors of 2, arranged in a column-walking matrix
    # view, over two batched 6x8 row-major matrices
    mem = tla.make_layout((8, 6, 2), (1, 8, 48))
    mat = tla.make_layout(((2, 4), 6, 2), ((1, 2), 8, 48))
    vec = tla.make_layout((2, 48), (1, 2))
    chain = tla.composition(tla.composition(mem, mat), vec)
    want = L.Composition(L.Composition(L.Layout((8, 6, 2), (1, 8, 48)),
                                       L.Layout(((2, 4), 6, 2), ((1, 2), 8, 48))),
                         L.Layout((2, 48), (1, 2))).table()
    assert _dev_table(chain) == want
    d = tla.logical_divide_modes(tla.make_layout(*sm80), (8, 4))
    assert _dev_table(d) == L.divide_modes(L.Layout(*sm80), (8, 4)).table()
    p = tla.logical_product(tla.make_layout((4, 8), (8, 1)), tla.make_layout(3, 32))
    assert _dev_table(p) == L.logical_product(L.Layout((4, 8), (8, 1)), L.Layout(3, 32)).table()
    c = tla.coalesce(tla.make_layout(((2, 2), 4, 1, 3), ((1, 2), 4, 7, 16)))
    assert _dev_table(c) == L.Layout(((2, 2), 4, 1, 3), ((1, 2), 4, 7, 16)).table()


def test_composed_tiled_view_at_scale():
    """A 512x512 row-major matrix seen as 16x16 tiles of 32x32, tile row
    fastest: the closed form from tla_composition, evaluated on the device
    over all 2^18 entries, equals A(B(i)) computed one entry at a time."""
    A = tla.make_layout((512, 512), (512, 1))
    B = tla.make_layout(((32, 32), (16, 16)), ((1, 512), (32, 16384)))
    R = tla.composition(A, B)
    got = _dev_table(R)
    a, b = L.Layout((512, 512), (512, 1)), L.Layout(((32, 32), (16, 16)), ((1, 512), (32, 16384)))
    rng = random.Random(4)
    for i in rng.sample(range(len(got)), 4096) + [0, len(got) - 1]:
        assert got[i] == a(b(i))
    # and the device's pointwise composition agrees everywhere
    assert got == _dev_table(A, B)


# -------------------------------------------------- thread-map variants on device

def _map_eval_ex(R, C, T, V, I, contig, G, shift, rows, cols):
    n = T * V * I
    idx = torch.full((n,), -1, dtype=torch.int64, device="cuda")
    val = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    tla.thread_map_eval_ex(R, C, T, V, I, contig, G, shift, rows, cols, idx, val)
    torch.cuda.synchronize()
    return idx.cpu().tolist(), val.cpu().tolist()


VARIANTS = [  # (R, C, T, V, I, contig, threads_per_row, swizzle_shift)
    (64, 64, 128, 4, 8, 1, 16, -1), (64, 64, 128, 4, 8, 1, 8, -1), (64, 64, 128, 4, 8, 1, 4, -1),
    (64, 64, 128, 4, 8, 1, 16, 0), (64, 64, 128, 4, 8, 1, 8, 2), (64, 64, 128, 4, 8, 0, 8, 1),
    (256, 8, 256, 1, 8, 1, 0, 1),            # the GEMM slab's swizzled copy
    (128, 64, 256, 8, 4, 1, 4, 1), (32, 128, 64, 8, 8, 1, 4, 0), (16, 16, 16, 2, 8, 1, 2, 1),
]


@pytest.mark.parametrize("R,C,T,V,I,contig,G,shift", VARIANTS)
def test_thread_map_variants_on_device(R, C, T, V, I, contig, G, shift):
    tm = L.StripMinedThreadMap(R, C, T, V, I, contig, threads_per_row=G, swizzle_shift=shift)
    for rows, cols in [(R, C), (R - 1, C - 3), (R // 2 + 1, 1)]:
        idx, val = _map_eval_ex(R, C, T, V, I, contig, G, shift, rows, cols)
        assert idx == tm.table()
        want = [0] * (T * V * I)
        for it in range(I):
            for v in range(V):
                for t in range(T):
                    want[t + T * (v + V * it)] = int(tm.valid(t, it, v, rows, cols))
        assert val == want
