// copy.hpp -- thread -> tile-coordinate maps for tiled global-memory copies.
//
// The strip-mined pitch-linear thread map (PitchLinearStripminedThreadMap
// walk-through, lpnh.cn/news/2469163, sections 2.1, 3.1-3.4, 4.2): an R x C
// tile is copied by T threads, each moving V contiguous elements per access
// and I accesses in all.  Threads are laid out contiguous-dimension first:
// G = Q/V threads share one strided position (Q = contiguous extent), so
// consecutive threads touch consecutive addresses, and iteration `it` moves a
// thread by the row stride S = P/I (P = strided extent):
//
//     contiguous = (t mod G)*V + v,   strided = t div G + it*S,
//     tile equation R*C == T*V*I,     S == T/G.
//
// contiguous_dim 1 is the page's row-contiguous map; 0 is its column-major
// variant (section 3.4) with the roles of rows and columns swapped.  The
// predicate (section 4.2) keeps an element only if it lies inside the part
// of the tile that exists; this library checks it per element.
//
// On gfx950 a wavefront is 64 threads: with G a divisor of 64 one wave reads
// 64/G whole strided positions per iteration.
#pragma once

#include "layout.hpp"

namespace tla {

struct StripMinedMap {
  int R, C, T, V, I, contig;
  int P, Q, G, S;  // strided extent, contiguous extent, column groups, row stride

  TLA_HD constexpr StripMinedMap(int R_, int C_, int T_, int V_, int I_, int contig_ = 1)
      : R(R_), C(C_), T(T_), V(V_), I(I_), contig(contig_),
        P(contig_ ? R_ : C_), Q(contig_ ? C_ : R_),
        G(V_ > 0 ? (contig_ ? C_ : R_) / V_ : 0),
        S(I_ > 0 ? (contig_ ? R_ : C_) / I_ : 0) {}

  // Every condition under which the map is a bijection onto the tile.
  TLA_HD constexpr bool well_formed() const {
    return R > 0 && C > 0 && T > 0 && V > 0 && I > 0 &&
           (int64_t)R * C == (int64_t)T * V * I && Q % V == 0 && G > 0 && T % G == 0 &&
           P % I == 0 && S == T / G;
  }

  TLA_HD constexpr int strided(int t, int it) const { return t / G + it * S; }
  TLA_HD constexpr int contiguous(int t, int v) const { return (t % G) * V + v; }
  TLA_HD constexpr int row(int t, int it, int v) const {
    return contig ? strided(t, it) : contiguous(t, v);
  }
  TLA_HD constexpr int col(int t, int it, int v) const {
    return contig ? contiguous(t, v) : strided(t, it);
  }
  // Tile index: row*C + col (row-contiguous) or row + col*R (column-contiguous).
  TLA_HD constexpr int index(int t, int it, int v) const {
    return contig ? row(t, it, v) * C + col(t, it, v) : row(t, it, v) + col(t, it, v) * R;
  }
  TLA_HD constexpr bool valid(int t, int it, int v, int64_t rows, int64_t cols) const {
    return row(t, it, v) < rows && col(t, it, v) < cols;
  }
  // The map as a thread/value layout ((G, T/G), (V, I)) : ((V, Q), (1, S*Q)),
  // stored flat; its 1-D index is t + T*(v + V*it).
  TLA_HD constexpr Layout<4, int> tv_layout() const {
    return Layout<4, int>{{G, T / G, V, I}, {V, Q, 1, S * Q}};
  }
};

}  // namespace tla
