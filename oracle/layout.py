"""Scalar layout evaluator -- the oracle for the layout algebra, the thread
maps and the layout-driven transpose.

Test infrastructure only (see the package docstring).  Pure Python, one
integer at a time, written for readability rather than speed.

Definitions followed (page titles and sections; no code is taken from them):

* "Advanced CUTLASS Architecture and Kernel Optimization" (oboe.com),
  section "The Algebra of Layouts": a Layout is a pair (Shape, Stride) of
  integer tuples and maps a coordinate to an index by the dot product of
  coordinate and stride (crd2idx).  The 4x8 row-major example has stride
  (8, 1).
* same page, "Functional Composition": A o B is the function c -> A(B(c)).
* same page, "Advanced Layout Operations": logical_divide splits one mode
  into a mode for the position inside a tile and a mode for the tile; 1024
  elements by 128 gives 8 tiles of 128.  logical_product concatenates shapes
  and strides.
* "CUTLASS / CuTe 主线" (hpc.payai.win/cutlass), "ldmatrix 指令与 CuTe TV
  Layout 映射", Parts 1-3: the lane tables of ldmatrix .x1 / .x4 and the
  hierarchical SM80 A-operand TV layout, whose column-major index m + 16k
  and Thread 0's printed values fix that a 1-D index walks a multi-mode
  shape colexicographically (first mode fastest).
* "什么是 CuTe ?" (GPU Glossary zh, 4.21), the transpose kernel: row-major
  and column-major layouts over one shape, tiled_divide by a 32x32 block,
  a slice by block index, local_partition by an 8x32 row-major thread
  layout.
* the PitchLinearStripminedThreadMap walk-through (lpnh.cn/news/2469163),
  sections 2.1, 3.1-3.2 and 4.2: the strip-mined thread map
  (tid, iteration) -> (row, column) and its predicate.
"""
from math import prod


# ------------------------------------------------------------------ tuples

def is_int(x) -> bool:
    return isinstance(x, int) and not isinstance(x, bool)


def size(shape) -> int:
    """Number of coordinates of a (possibly nested) shape: product of leaves."""
    if is_int(shape):
        return shape
    return prod(size(s) for s in shape)


def flatten(t):
    """Leaves of a nested tuple, in order."""
    if is_int(t):
        return (t,)
    out = ()
    for s in t:
        out += flatten(s)
    return out


def congruent(a, b) -> bool:
    if is_int(a) or is_int(b):
        return is_int(a) and is_int(b)
    return len(a) == len(b) and all(congruent(x, y) for x, y in zip(a, b))


# ----------------------------------------------------- coordinates <-> index

def idx2crd(i: int, shape):
    """Natural coordinate of 1-D index ``i`` in ``shape``, colexicographic
    (the first mode varies fastest), recursively inside nested modes.

    Reading: the pages never state the order in words; the column-major
    index m + 16k of the SM80 ALayout and Thread 0's value order (CUTLASS /
    CuTe 主线, ldmatrix section, Part 3) fix it as colexicographic.
    """
    if is_int(shape):
        if not 0 <= i < max(shape, 1):
            raise IndexError("index %d outside mode of extent %d" % (i, shape))
        return i
    if not 0 <= i < max(size(shape), 1):
        raise IndexError("index %d outside shape %r" % (i, shape))
    crd = []
    for s in shape:
        n = size(s)
        crd.append(idx2crd(i % n, s))
        i //= n
    return tuple(crd)


def crd2idx(crd, shape, stride) -> int:
    """Index of coordinate ``crd``: the dot product of coordinate and stride
    ("The Algebra of Layouts").  An integer given for a nested mode is first
    turned into that mode's natural coordinate (colexicographic)."""
    if is_int(shape):
        if not is_int(crd):
            raise TypeError("tuple coordinate for a scalar mode")
        return crd * stride
    if is_int(crd):
        crd = idx2crd(crd, shape)
    if len(crd) != len(shape):
        raise ValueError("coordinate rank %d != shape rank %d" % (len(crd), len(shape)))
    return sum(crd2idx(c, s, d) for c, s, d in zip(crd, shape, stride))


class Layout:
    """A (Shape, Stride) pair viewed as a function from coordinates to an
    integer index."""

    def __init__(self, shape, stride):
        if not congruent(shape, stride):
            raise ValueError("shape %r and stride %r are not congruent" % (shape, stride))
        self.shape, self.stride = shape, stride

    def size(self) -> int:
        return size(self.shape)

    def __call__(self, *crd) -> int:
        c = crd[0] if len(crd) == 1 else tuple(crd)
        return crd2idx(c, self.shape, self.stride)

    def table(self):
        """[L(0), L(1), ..., L(size-1)] over the colexicographic order."""
        return [self(i) for i in range(self.size())]

    def __repr__(self):
        return "Layout(%r : %r)" % (self.shape, self.stride)


def row_major(shape) -> Layout:
    """Flat shape, last mode contiguous: stride of mode i = product of the
    extents after it (the 4x8 example has stride (8, 1))."""
    stride, acc = [], 1
    for s in reversed(shape):
        stride.append(acc)
        acc *= s
    return Layout(tuple(shape), tuple(reversed(stride)))


def col_major(shape) -> Layout:
    """Flat shape, first mode contiguous: stride of mode i = product of the
    extents before it."""
    stride, acc = [], 1
    for s in shape:
        stride.append(acc)
        acc *= s
    return Layout(tuple(shape), tuple(stride))


# -------------------------------------------------------------- composition

class Composition:
    """A o B, evaluated pointwise: c -> A(B(c)) ("Functional Composition").

    B's value is handed to A as a 1-D index, so it must lie in
    [0, size(A)); A takes it through its colexicographic idx2crd.  The domain
    is B's domain.
    """

    def __init__(self, A: Layout, B: Layout):
        self.A, self.B = A, B

    def size(self) -> int:
        return self.B.size()

    def __call__(self, *crd) -> int:
        inner = self.B(*crd)
        if not 0 <= inner < self.A.size():
            raise IndexError("B(c) = %d outside A's domain [0,%d)" % (inner, self.A.size()))
        return self.A(inner)

    def table(self):
        return [self(i) for i in range(self.size())]


# ------------------------------------------------------------------ divides

def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class Divided:
    """logical_divide of a flat layout by a tile shape, as a function.

    Each mode i of extent n_i is split into (e, t): e < tile_i is the
    position inside the tile and t < ceil(n_i / tile_i) the tile index, and
    the element at (e, t) is the original element at coordinate
    e + tile_i * t ("Advanced Layout Operations": one mode becomes a mode for
    the tile and a mode inside it; 1024 by 128 gives 8 tiles of 128).

    Mode order (reading): (inside-tile, tile-index).  The page lists the two
    modes the other way round; the function is the same, so tests compare
    by coordinate, never by the 1-D order.

    When the tile does not divide the extent, the last tile reaches past the
    end; ``in_range`` tells which coordinates are real elements (the
    predicate of the thread-map walk-through, section 4.2).
    """

    def __init__(self, L: Layout, tile):
        shape = (L.shape,) if is_int(L.shape) else tuple(L.shape)
        stride = (L.stride,) if is_int(L.stride) else tuple(L.stride)
        tile = (tile,) if is_int(tile) else tuple(tile)
        if len(tile) != len(shape) or not all(is_int(s) for s in shape):
            raise ValueError("one tile extent per flat mode is required")
        if any(t <= 0 for t in tile):
            raise ValueError("tile extents must be positive")
        self.L, self.extent, self.ustride, self.tile = L, shape, stride, tile
        self.rest = tuple(ceil_div(n, t) for n, t in zip(shape, tile))
        self.shape = tuple((t, r) for t, r in zip(tile, self.rest))

    def size(self) -> int:
        return size(self.shape)

    def original_coord(self, crd):
        """((e0,t0), (e1,t1), ...) -> (e0 + tile0*t0, e1 + tile1*t1, ...)."""
        if is_int(crd):
            crd = idx2crd(crd, self.shape)
        if len(self.shape) == 1 and len(crd) == 2 and is_int(crd[0]):
            crd = (crd,)
        out = []
        for (e, t), T, R in zip(crd, self.tile, self.rest):
            if not (0 <= e < T and 0 <= t < R):
                raise IndexError("coordinate outside the divided shape")
            out.append(e + T * t)
        return tuple(out)

    def in_range(self, crd) -> bool:
        return all(c < n for c, n in zip(self.original_coord(crd), self.extent))

    def __call__(self, *crd) -> int:
        c = crd[0] if len(crd) == 1 else tuple(crd)
        oc = self.original_coord(c)
        # A flat mode maps its coordinate linearly, so the layout's value is
        # defined (and used by the padded last tile) even past the extent.
        return sum(x * d for x, d in zip(oc, self.ustride))


def logical_divide(L: Layout, tile) -> Divided:
    return Divided(L, tile)


class TiledDivided:
    """tiled_divide: logical_divide, then the inside-tile modes gathered into
    mode 0: coordinate ((e0, e1, ...), t0, t1, ...).  Reading of its use in
    "什么是 CuTe ?" (transpose kernel), where a tile is picked by
    ``(make_coord(_,_), blockIdx.x, blockIdx.y)``; the page defines the
    operation only through that use."""

    def __init__(self, L: Layout, tile):
        self.d = Divided(L, tile)
        self.shape = (tuple(self.d.tile),) + tuple(self.d.rest)

    def size(self) -> int:
        return self.d.size()

    def _to_divided(self, crd):
        if is_int(crd):
            crd = idx2crd(crd, self.shape)
        inner, tiles = crd[0], crd[1:]
        if is_int(inner):
            inner = idx2crd(inner, self.shape[0])
        return tuple((e, t) for e, t in zip(inner, tiles))

    def in_range(self, crd) -> bool:
        return self.d.in_range(self._to_divided(crd))

    def __call__(self, *crd) -> int:
        c = crd[0] if len(crd) == 1 else tuple(crd)
        return self.d(self._to_divided(c))

    def tile_at(self, *tile_idx):
        """The slice (make_coord(_,...), t0, t1, ...): a function of the
        inside-tile coordinate."""
        return lambda *e: self((tuple(e),) + tuple(tile_idx))


def tiled_divide(L: Layout, tile) -> TiledDivided:
    return TiledDivided(L, tile)


# ---------------------------------------------------- product and nested divide

def modes_of(L: Layout):
    """Top-level modes of L as (shape, stride) pairs (an integer shape is one
    mode)."""
    if is_int(L.shape):
        return [(L.shape, L.stride)]
    return list(zip(L.shape, L.stride))


def logical_product(L: Layout, M: Layout) -> Layout:
    """logical_product in the reading of "Advanced Layout Operations": the
    shape and the stride of the result are the concatenations of the
    inputs' (L's modes first, then M's)."""
    ml, mm = modes_of(L), modes_of(M)
    return Layout(tuple(s for s, _ in ml + mm), tuple(d for _, d in ml + mm))


class DividedModes:
    """logical_divide of every top-level mode of L, nested modes included.

    Mode i (shape s_i, stride d_i, size n_i) and tile t_i become two modes,
    the position e < t_i inside the tile and the tile index
    q < ceil(n_i / t_i), and stand for the element at 1-D position
    e + t_i * q of mode i, taken through that mode's own colexicographic
    idx2crd ("Advanced Layout Operations": one mode becomes a tile mode and a
    mode inside the tile).  The result's modes are ordered
    (inside_0, index_0, inside_1, index_1, ...).

    A flat mode n:d maps its coordinate linearly, so a ragged last tile
    keeps the value x*d past the end (as Divided does); for a nested mode
    the tile must divide the mode's size.
    """

    def __init__(self, L: Layout, tile):
        self.modes = modes_of(L)
        tile = (tile,) if is_int(tile) else tuple(tile)
        if len(tile) != len(self.modes) or any(t <= 0 for t in tile):
            raise ValueError("one positive tile extent per mode is required")
        self.tile = tile
        self.rest = []
        for (s, _), t in zip(self.modes, tile):
            n = size(s)
            if not is_int(s) and n % t:
                raise ValueError("a nested mode needs a tile dividing its size")
            self.rest.append(ceil_div(n, t))
        self.shape = tuple(x for t, r in zip(tile, self.rest) for x in (t, r))

    def size(self) -> int:
        return size(self.shape)

    def __call__(self, i: int) -> int:
        crd = idx2crd(i, self.shape)
        total = 0
        for k, ((s, d), t) in enumerate(zip(self.modes, self.tile)):
            x = crd[2 * k] + t * crd[2 * k + 1]
            total += x * d if is_int(s) else crd2idx(idx2crd(x, s), s, d)
        return total

    def table(self):
        return [self(i) for i in range(self.size())]


def divide_modes(L: Layout, tile) -> DividedModes:
    return DividedModes(L, tile)


# ---------------------------------------------------------- local_partition

def thread_coord(thr_layout: Layout, tid: int):
    """The coordinate c with thr_layout(c) == tid, found by search (the thread
    layout must be injective on its domain)."""
    hits = [idx2crd(i, thr_layout.shape) for i in range(thr_layout.size())
            if thr_layout(i) == tid]
    if len(hits) != 1:
        raise ValueError("thread %d has %d coordinates in %r" % (tid, len(hits), thr_layout))
    return hits[0]


def local_partition(tile_fn, tile_shape, thr_layout: Layout, tid: int):
    """The elements of a tile owned by thread ``tid``, as a list of tile
    coordinates in the thread's own colexicographic value order.

    Reading of the transpose kernel in "什么是 CuTe ?": with a tile of
    shape (R, C) and a thread layout of shape (tR, tC), thread tid sits at
    thread coordinate (r, c) and owns the elements (r + tR*i, c + tC*j) for
    i < R/tR, j < C/tC.  ``tile_fn`` maps a tile coordinate to the index
    the caller wants (it is applied to every owned coordinate).
    """
    r0, c0 = thread_coord(thr_layout, tid)
    tR, tC = thr_layout.shape
    R, C = tile_shape
    if R % tR or C % tC:
        raise ValueError("thread layout does not divide the tile")
    # colexicographic over the thread's own (i, j): i fastest
    owned = [(r0 + tR * i, c0 + tC * j) for j in range(C // tC) for i in range(R // tR)]
    return [tile_fn(*rc) for rc in owned]


# ------------------------------------------------------------ thread maps

class StripMinedThreadMap:
    """The strip-mined pitch-linear thread map (walk-through, sections 2.1,
    3.1, 3.2): an R x C tile, T threads, V contiguous elements per access,
    I iterations per thread.

      tile equation     R*C == T*V*I            (section 2.1)
      column groups     G = C / V               (section 3.1)
      column            col = (t mod G)*V + v   (section 3.1)
      row anchor        t div G                 (section 3.1)
      row               row = t div G + it*S    (section 3.1)
      row stride        S = R / I               (reading: fixed by the tile)

    ``contiguous_dim`` 1 is the page's map (columns contiguous).  0 is the
    column-major variant of section 3.4 with the roles of rows and columns
    swapped: rows are split into groups of V and the iterations step along
    columns.

    Two options of the same walk-through, off by default:

    * ``threads_per_row`` (section 2.2: the base map takes a parameter that
      overrides the default thread distribution).  Reading: G threads share
      one row instead of C/V; each thread then makes Ic = (C/V)/G passes
      along the row (innermost) per row step, so iteration it is the pass
      it mod Ic of row step it div Ic:
        column group = t mod G + G*(it mod Ic),  row = t div G + (it div Ic)*S,
      with S = T/G the row stride and R == S*(I/Ic).
    * ``swizzle_shift`` (section 5.3: a map that exchanges bits of the
      thread-to-address mapping to spread bank conflicts).  Reading: the
      column group is XORed with (row >> shift) mod (C/V), C/V a power of
      two -- every row's groups are permuted among themselves.
    """

    def __init__(self, R, C, T, V, I, contiguous_dim=1, threads_per_row=0, swizzle_shift=-1):
        if min(R, C, T, V, I) <= 0:
            raise ValueError("all extents must be positive")
        if R * C != T * V * I:
            raise ValueError("tile equation R*C == T*V*I violated")
        self.R, self.C, self.T, self.V, self.I = R, C, T, V, I
        self.contig = contiguous_dim
        P, Q = (R, C) if contiguous_dim == 1 else (C, R)  # P strided, Q contiguous
        if Q % V:
            raise ValueError("vector width must divide the contiguous extent")
        self.groups = Q // V
        self.G = threads_per_row if threads_per_row > 0 else self.groups
        if self.groups % self.G:
            raise ValueError("threads per row must divide the column groups")
        self.Ic = self.groups // self.G
        if T % self.G or I % self.Ic:
            raise ValueError("threads do not tile the strided extent")
        self.S = T // self.G
        if P != self.S * (I // self.Ic):
            raise ValueError("row stride times row steps differs from the strided extent")
        if swizzle_shift >= 0 and self.groups & (self.groups - 1):
            raise ValueError("a swizzle needs a power-of-two number of column groups")
        self.shift = swizzle_shift

    def coord(self, t, it, v):
        """(row, col) visited by thread t, iteration it, vector lane v."""
        if not (0 <= t < self.T and 0 <= it < self.I and 0 <= v < self.V):
            raise IndexError("(t, it, v) out of range")
        strided = t // self.G + (it // self.Ic) * self.S
        group = t % self.G + self.G * (it % self.Ic)
        if self.shift >= 0:
            group ^= (strided >> self.shift) % self.groups
        contiguous = group * self.V + v
        return (strided, contiguous) if self.contig == 1 else (contiguous, strided)

    def index(self, t, it, v):
        """The coordinate as an index into the tile: row*C + col for the
        row-contiguous map, row + col*R for the column-contiguous one."""
        r, c = self.coord(t, it, v)
        return r * self.C + c if self.contig == 1 else r + c * self.R

    def valid(self, t, it, v, M, N):
        """Predicate, per element: the element lies inside the (M, N) part of
        the tile that exists (section 4.2 checks row < M and the column
        against N; reading: every element of the vector is checked)."""
        r, c = self.coord(t, it, v)
        return r < M and c < N

    def valid_page_form(self, t, it, M, N):
        """Section 4.2's own form: row < M and the vector's first column < N
        (row-contiguous map only)."""
        r, c = self.coord(t, it, 0)
        return r < M and c < N

    def tv_layout(self) -> Layout:
        """The same map as a (thread, value) layout: thread modes (G, T/G),
        value modes (V, I), into the tile index.  Reading (the page states
        the map as formulas only): strides ((V, Q), (1, S*Q)) with Q the
        contiguous extent; with several passes per row the iteration mode
        splits into (Ic, I/Ic) with strides (G*V, S*Q).  A swizzled map is
        not a shape/stride layout."""
        if self.shift >= 0:
            raise ValueError("a swizzled map has no shape/stride form")
        Q = self.C if self.contig == 1 else self.R
        if self.Ic == 1:
            return Layout(((self.G, self.T // self.G), (self.V, self.I)),
                          ((self.V, Q), (1, self.S * Q)))
        return Layout(((self.G, self.T // self.G), (self.V, self.Ic, self.I // self.Ic)),
                      ((self.V, Q), (1, self.G * self.V, self.S * Q)))

    def table(self):
        """out[t + T*(v + V*it)] = index(t, it, v): the TV layout's 1-D table
        with the thread index fastest."""
        out = [0] * (self.T * self.V * self.I)
        for it in range(self.I):
            for v in range(self.V):
                for t in range(self.T):
                    out[t + self.T * (v + self.V * it)] = self.index(t, it, v)
        return out


# ------------------------------------------------- printed operand tables

def ldmatrix_x1(lane: int):
    """ldmatrix .x1 over one 8x8 fp16 matrix: lane -> its two (row, col)
    (CUTLASS / CuTe 主线, ldmatrix section, Part 1): row = lane / 4,
    first column = (lane % 4) * 2, two neighbouring elements."""
    r, c = lane // 4, (lane % 4) * 2
    return [(r, c), (r, c + 1)]


def ldmatrix_x4(t: int):
    """ldmatrix .x4 for the 16x16 A operand (same page, Part 2): thread t's
    registers d0..d3, two halves each, as (row, col) in order
    d0.lo d0.hi d1.lo ... d3.hi.  g = t/4, c = 2(t%4); d0 = A[g][c..c+1],
    d1 = A[g+8][c..], d2 = A[g][c+8..], d3 = A[g+8][c+8..]."""
    g, c = t // 4, (t % 4) * 2
    out = []
    for j in range(4):
        for h in range(2):
            out.append((g + 8 * (j % 2), c + h + 8 * (j // 2)))
    return out


SM80_A_LAYOUT = Layout(((4, 8), (2, 2, 2)), ((32, 1), (16, 8, 128)))
"""SM80 16x8x16 A operand, (T32, V8) -> (M16, K16), index m + 16k
(same page, Part 3)."""


def sm80_a_coord(t: int, v: int):
    """(m, k) of thread t's value v under SM80_A_LAYOUT."""
    idx = SM80_A_LAYOUT((t, v))
    return (idx % 16, idx // 16)


def xor_swizzle_chunk(row: int, chunk: int, bits: int = 3) -> int:
    """The shared-memory swizzle as the ldmatrix section (Part 4) states it:
    the row number is XORed into the 16-byte chunk index, so the 8 rows one
    ldmatrix reads fall into different banks.  ``bits`` chunk-index bits;
    the row enters modulo 2**bits."""
    m = (1 << bits) - 1
    return (chunk & m) ^ (row & m)
