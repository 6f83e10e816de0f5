// layout.hpp -- shape/stride layout algebra, usable in constant expressions
// on the host and inside gfx950 kernels.
//
// A Layout is a pair of integer tuples, Shape and Stride; it maps a
// coordinate to an index by the dot product of coordinate and stride, and a
// 1-D index to a coordinate colexicographically (first mode fastest).  When
// a layout is a compile-time constant every divide and modulo below folds
// into shifts and masks, so a kernel written against layouts pays nothing
// at run time for them.
//
// Sources: "Advanced CUTLASS Architecture and Kernel Optimization"
// (oboe.com), sections "The Algebra of Layouts" (Shape, Stride, crd2idx),
// "Functional Composition" (A o B) and "Advanced Layout Operations"
// (logical_divide); "什么是 CuTe ?" (GPU Glossary zh, 4.21) for
// tiled_divide, slicing a tile by block index and local_partition; "CUTLASS
// / CuTe 主线" (hpc.payai.win/cutlass), ldmatrix section Part 3, for the
// colexicographic order of multi-mode indices.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#define TLA_HD __host__ __device__ __forceinline__

namespace tla {

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. N-1, expanded at
// compile time, so register arrays indexed by i never need addressable
// (scratch) storage.
template <int N, typename F>
TLA_HD constexpr void static_for(F&& f) {
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
  }(std::make_integer_sequence<int, N>{});
}

template <int R, typename I = int>
struct Coord {
  I v[R];
  TLA_HD constexpr I operator[](int i) const { return v[i]; }
  TLA_HD constexpr I& operator[](int i) { return v[i]; }
};

// A flat layout of rank R.  Nested layouts with one level of nesting are
// stored flat, leaf by leaf: a 1-D index walks the leaves colexicographically
// either way, so only the grouping of leaves into modes differs.
template <int R, typename I = int>
struct Layout {
  I shape[R];
  I stride[R];

  TLA_HD constexpr I size() const {
    I s = 1;
    for (int i = 0; i < R; ++i) s *= shape[i];
    return s;
  }

  // crd2idx: dot product of coordinate and stride.
  TLA_HD constexpr I operator()(const Coord<R, I>& c) const {
    I idx = 0;
    for (int i = 0; i < R; ++i) idx += c.v[i] * stride[i];
    return idx;
  }

  // idx2crd (colexicographic), then crd2idx.
  TLA_HD constexpr I operator()(I idx) const { return (*this)(idx2crd(idx)); }

  TLA_HD constexpr Coord<R, I> idx2crd(I idx) const {
    Coord<R, I> c{};
    for (int i = 0; i < R; ++i) {
      c.v[i] = idx % shape[i];
      idx /= shape[i];
    }
    return c;
  }
};

template <typename I = int>
TLA_HD constexpr Layout<2, I> make_layout(I s0, I s1, I d0, I d1) {
  return Layout<2, I>{{s0, s1}, {d0, d1}};
}

// Strides of a compact row-major (last mode contiguous) / column-major (first
// mode contiguous) matrix with a pitch: the pitch is part of the tensor
// layout, never derived from the column count.
template <typename I = int>
TLA_HD constexpr Layout<2, I> row_major(I rows, I cols, I ld) {
  return Layout<2, I>{{rows, cols}, {ld, 1}};
}
template <typename I = int>
TLA_HD constexpr Layout<2, I> col_major(I rows, I cols, I ld) {
  return Layout<2, I>{{rows, cols}, {1, ld}};
}

// The coordinate of `idx` under a compact layout (a bijection of its domain
// onto [0, size) with positive strides): each mode's coordinate is
// (idx / stride) mod extent.  Used to place a thread inside a thread layout.
template <int R, typename I>
TLA_HD constexpr Coord<R, I> compact_inverse(const Layout<R, I>& L, I idx) {
  Coord<R, I> c{};
  for (int i = 0; i < R; ++i) c.v[i] = (idx / L.stride[i]) % L.shape[i];
  return c;
}

// Pointwise composition A o B: i -> A(B(i)); B's value is a 1-D index into
// A's (colexicographic) domain.
template <int RA, int RB, typename I>
struct Composition {
  Layout<RA, I> A;
  Layout<RB, I> B;
  TLA_HD constexpr I size() const { return B.size(); }
  TLA_HD constexpr I operator()(I i) const { return A(B(i)); }
};
template <int RA, int RB, typename I>
TLA_HD constexpr Composition<RA, RB, I> compose(const Layout<RA, I>& A, const Layout<RB, I>& B) {
  return Composition<RA, RB, I>{A, B};
}

TLA_HD constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// logical_divide of a flat layout by a tile shape.  Mode i (extent n, stride
// d) becomes the leaf pair (tile_i, ceil(n/tile_i)) : (d, d*tile_i): the
// position inside the tile first, the tile index second.
template <int R, typename I>
TLA_HD constexpr Layout<2 * R, I> logical_divide(const Layout<R, I>& L, const I (&tile)[R]) {
  Layout<2 * R, I> out{};
  for (int i = 0; i < R; ++i) {
    out.shape[2 * i] = tile[i];
    out.shape[2 * i + 1] = (I)ceil_div(L.shape[i], tile[i]);
    out.stride[2 * i] = L.stride[i];
    out.stride[2 * i + 1] = L.stride[i] * tile[i];
  }
  return out;
}

// tiled_divide: the same leaves reordered as ((tile_0, ..., tile_{R-1}),
// rest_0, ..., rest_{R-1}) -- all inside-tile leaves first (mode 0), then one
// mode per tile index.
template <int R, typename I>
TLA_HD constexpr Layout<2 * R, I> tiled_divide(const Layout<R, I>& L, const I (&tile)[R]) {
  Layout<2 * R, I> d = logical_divide(L, tile), out{};
  for (int i = 0; i < R; ++i) {
    out.shape[i] = d.shape[2 * i];
    out.stride[i] = d.stride[2 * i];
    out.shape[R + i] = d.shape[2 * i + 1];
    out.stride[R + i] = d.stride[2 * i + 1];
  }
  return out;
}

// A tensor view: a base offset plus a layout.  Slicing and partitioning
// return views of the same memory.
template <int R, typename I = int>
struct View {
  I offset;
  Layout<R, I> layout;
  TLA_HD constexpr I operator()(const Coord<R, I>& c) const { return offset + layout(c); }
  TLA_HD constexpr I operator()(I idx) const { return offset + layout(idx); }
};

// The tile (make_coord(_, _), t_0, t_1) of a rank-2 tiled_divide result:
// fixes the two tile-index modes, keeps the inside-tile modes.
template <typename I>
TLA_HD constexpr View<2, I> tile_slice(const Layout<4, I>& td, I t0, I t1) {
  return View<2, I>{t0 * td.stride[2] + t1 * td.stride[3],
                    Layout<2, I>{{td.shape[0], td.shape[1]}, {td.stride[0], td.stride[1]}}};
}

// local_partition: thread `tid` of a rank-2 thread layout sits at thread
// coordinate (r, c) and owns the tile elements (r + tR*i, c + tC*j),
// i < R/tR, j < C/tC -- a strided sub-view of the tile.
template <typename I>
TLA_HD constexpr View<2, I> local_partition(const View<2, I>& tile, const Layout<2, I>& thr, I tid) {
  Coord<2, I> tc = compact_inverse(thr, tid);
  I tR = thr.shape[0], tC = thr.shape[1];
  View<2, I> out{};
  out.offset = tile.offset + tc.v[0] * tile.layout.stride[0] + tc.v[1] * tile.layout.stride[1];
  out.layout.shape[0] = tile.layout.shape[0] / tR;
  out.layout.shape[1] = tile.layout.shape[1] / tC;
  out.layout.stride[0] = tile.layout.stride[0] * tR;
  out.layout.stride[1] = tile.layout.stride[1] * tC;
  return out;
}

// ---------------------------------------------------------------- swizzle
// XOR swizzle of 16-byte chunks inside an LDS row of `kChunks` chunks: the
// physical chunk of logical chunk c in row r is c ^ f(r).  f takes row bits
// above `kRowShift`, so the rows a group of lanes reads together at one
// logical chunk land on distinct banks.  An involution in c for every row.
template <int kChunks, int kRowShift>
struct XorSwizzle {
  static_assert((kChunks & (kChunks - 1)) == 0, "power-of-two chunk count");
  TLA_HD static constexpr int f(int row) { return (row >> kRowShift) & (kChunks - 1); }
  TLA_HD static constexpr int chunk(int row, int c) { return c ^ f(row); }
};

}  // namespace tla
