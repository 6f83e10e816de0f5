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
// Two further options of the same walk-through, both off by default:
//  * threads per row (section 2.2: a parameter that overrides the default
//    thread distribution).  Reading: with G < Q/V threads on one strided
//    position, a thread makes Ic = (Q/V)/G passes along the contiguous
//    dimension (innermost) for every step along the strided one:
//        group = (t mod G) + G*(it mod Ic),   strided = t div G + (it div Ic)*S,
//    with S = T/G and P == S*(I/Ic).  G = Q/V gives the map above.
//  * a swizzled map (section 5.3: exchange bits of the thread-to-address
//    mapping to spread bank conflicts).  Reading: the column group is XORed
//    with (strided >> shift) mod (Q/V), Q/V a power of two -- a permutation
//    of the groups of every strided position, so the map stays a bijection.
//    This is the permutation the GEMM's direct-to-LDS loads apply.
//
// On gfx950 a wavefront is 64 threads: with G a divisor of 64 one wave reads
// 64/G whole strided positions per iteration.
#pragma once

#include "layout.hpp"

namespace tla {

struct StripMinedMap {
  int R, C, T, V, I, contig;
  int P, Q, G, S;  // strided extent, contiguous extent, threads per position, row stride
  int Ic;          // passes along the contiguous dimension per strided step
  int shift;       // swizzle shift, -1 = no swizzle

  TLA_HD constexpr StripMinedMap(int R_, int C_, int T_, int V_, int I_, int contig_ = 1,
                                 int threads_per_row = 0, int swizzle_shift = -1)
      : R(R_), C(C_), T(T_), V(V_), I(I_), contig(contig_),
        P(contig_ ? R_ : C_), Q(contig_ ? C_ : R_),
        G(threads_per_row > 0 ? threads_per_row : (V_ > 0 ? (contig_ ? C_ : R_) / V_ : 0)),
        S(0), Ic(0), shift(swizzle_shift) {
    const int groups = V_ > 0 ? Q / V_ : 0;
    Ic = G > 0 ? groups / G : 0;
    S = G > 0 ? T_ / G : 0;
  }

  // Every condition under which the map is a bijection onto the tile.
  TLA_HD constexpr bool well_formed() const {
    if (R <= 0 || C <= 0 || T <= 0 || V <= 0 || I <= 0 || G <= 0) return false;
    if ((int64_t)R * C != (int64_t)T * V * I || Q % V != 0) return false;
    const int groups = Q / V;
    if (groups % G != 0 || T % G != 0 || Ic <= 0 || I % Ic != 0) return false;
    if (P != S * (I / Ic)) return false;
    if (shift >= 0 && (shift > 30 || (groups & (groups - 1)) != 0)) return false;
    return true;
  }

  TLA_HD constexpr int strided(int t, int it) const { return t / G + (it / Ic) * S; }
  // Unswizzled, first-pass column of lane v (the common case G = Q/V).
  TLA_HD constexpr int contiguous(int t, int v) const { return (t % G) * V + v; }
  // Column group of (t, it): pass it mod Ic, swizzled by the strided position.
  TLA_HD constexpr int group(int t, int it) const {
    const int g = t % G + G * (it % Ic);
    return shift >= 0 ? g ^ ((strided(t, it) >> shift) & (Q / V - 1)) : g;
  }
  TLA_HD constexpr int row(int t, int it, int v) const {
    return contig ? strided(t, it) : group(t, it) * V + v;
  }
  TLA_HD constexpr int col(int t, int it, int v) const {
    return contig ? group(t, it) * V + v : strided(t, it);
  }
  // Tile index: row*C + col (row-contiguous) or row + col*R (column-contiguous).
  TLA_HD constexpr int index(int t, int it, int v) const {
    return contig ? row(t, it, v) * C + col(t, it, v) : row(t, it, v) + col(t, it, v) * R;
  }
  TLA_HD constexpr bool valid(int t, int it, int v, int64_t rows, int64_t cols) const {
    return row(t, it, v) < rows && col(t, it, v) < cols;
  }
  // The unswizzled map as a thread/value layout into the tile index,
  //   ((G, T/G), (V, I)) : ((V, Q), (1, S*Q))               when Ic == 1,
  //   ((G, T/G), (V, Ic, I/Ic)) : ((V, Q), (1, G*V, S*Q))   otherwise,
  // stored flat; its 1-D index is t + T*(v + V*it).
  TLA_HD constexpr Layout<4, int> tv_layout() const {
    return Layout<4, int>{{G, T / G, V, I}, {V, Q, 1, S * Q}};
  }
};

}  // namespace tla
