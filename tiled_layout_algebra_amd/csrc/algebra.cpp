// algebra.cpp -- host-side layout algebra on tla_layout descriptors:
// logical_product, coalesce, closed-form composition and the divide of
// nested modes.  Declarations and contracts are in include/tla.h.
//
// Following "Advanced CUTLASS Architecture and Kernel Optimization",
// "Functional Composition" (A o B is c -> A(B(c))) and "Advanced Layout
// Operations" (logical_divide splits a mode into a tile mode and an inside
// mode; logical_product concatenates shapes and strides).  The pages define
// composition pointwise; the closed form built here is the run of A's
// mixed-radix digits each leaf of B walks, and it is only returned when it
// reproduces the pointwise function exactly.
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "tla.h"

namespace {

// A descriptor's leaves, in order, with its mode structure.
struct Leaves {
  int n = 0;
  int64_t shape[TLA_MAX_LEAVES];
  int64_t stride[TLA_MAX_LEAVES];
};

// Structural checks shared by every entry point; the size must fit int64.
int read(const tla_layout* L, Leaves* f, int64_t* size) {
  if (!L || L->n_modes < 1 || L->n_modes > TLA_MAX_MODES) return TLA_ERR_INVALID_ARG;
  int n = 0;
  for (int i = 0; i < L->n_modes; ++i) {
    if (L->leaves[i] < 1 || L->leaves[i] > TLA_MAX_LEAVES) return TLA_ERR_INVALID_ARG;
    n += L->leaves[i];
  }
  if (n > TLA_MAX_LEAVES) return TLA_ERR_INVALID_ARG;
  int64_t s = 1;
  for (int i = 0; i < n; ++i) {
    if (L->shape[i] < 1 || s > INT64_MAX / L->shape[i]) return TLA_ERR_INVALID_ARG;
    s *= L->shape[i];
    f->shape[i] = L->shape[i];
    f->stride[i] = L->stride[i];
  }
  f->n = n;
  if (size) *size = s;
  return TLA_OK;
}

// First leaf index of each top-level mode.
void mode_starts(const tla_layout* L, int* first) {
  int k = 0;
  for (int i = 0; i < L->n_modes; ++i) {
    first[i] = k;
    k += L->leaves[i];
  }
}

// Drop extent-1 leaves and merge neighbours whose strides continue each
// other; a size-1 layout becomes the single leaf 1:0.
void coalesce_leaves(const Leaves& in, Leaves* out) {
  Leaves r;
  for (int i = 0; i < in.n; ++i) {
    if (in.shape[i] == 1) continue;
    int64_t next;
    if (r.n > 0 && !__builtin_mul_overflow(r.shape[r.n - 1], r.stride[r.n - 1], &next) &&
        in.stride[i] == next) {
      r.shape[r.n - 1] *= in.shape[i];
    } else {
      r.shape[r.n] = in.shape[i];
      r.stride[r.n] = in.stride[i];
      ++r.n;
    }
  }
  if (r.n == 0) {
    r.n = 1;
    r.shape[0] = 1;
    r.stride[0] = 0;
  }
  *out = r;
}

// Smallest and largest value of a layout (each leaf contributes between 0
// and (extent-1)*stride).  False on int64 overflow.
bool value_range(const Leaves& f, int64_t* lo, int64_t* hi) {
  int64_t a = 0, b = 0;
  for (int i = 0; i < f.n; ++i) {
    const int64_t e = f.shape[i] - 1, d = f.stride[i];
    if (e != 0 && (d > INT64_MAX / e || d < INT64_MIN / e)) return false;
    const int64_t span = e * d;
    if (span < 0) {
      if (a < INT64_MIN - span) return false;
      a += span;
    } else {
      if (b > INT64_MAX - span) return false;
      b += span;
    }
  }
  *lo = a;
  *hi = b;
  return true;
}

// Leaves of A o (s:d), appended to `out`.  A is coalesced (no extent-1
// leaves, at least one leaf), d > 0 and (s-1)*d < size(A).  The indices
// 0, d, ..., (s-1)d skip the leading modes whose extents multiply into d,
// then step by r = d / (those extents) through the next mode (r must divide
// it), carrying into the modes after it with stride 1 once that mode is
// used up; the last mode of A is unbounded.
int compose_leaf(const Leaves& A, int64_t s, int64_t d, Leaves* out) {
  auto emit = [&](int64_t shape, int64_t stride) {
    if (out->n == TLA_MAX_LEAVES) return false;
    out->shape[out->n] = shape;
    out->stride[out->n] = stride;
    ++out->n;
    return true;
  };
  if (s == 1) return emit(1, 0) ? TLA_OK : TLA_ERR_UNSUPPORTED;
  if (d == 0) return emit(s, 0) ? TLA_OK : TLA_ERR_UNSUPPORTED;
  int k = 0;
  int64_t r = d;
  while (k < A.n - 1 && r >= A.shape[k]) {
    if (r % A.shape[k] != 0) return TLA_ERR_UNSUPPORTED;
    r /= A.shape[k];
    ++k;
  }
  if (k < A.n - 1 && A.shape[k] % r != 0) return TLA_ERR_UNSUPPORTED;
  if (r > 1) {
    for (int i = k; i < A.n; ++i)
      if (A.stride[i] > INT64_MAX / r || A.stride[i] < INT64_MIN / r) return TLA_ERR_UNSUPPORTED;
  }
  int64_t rest = s;
  for (;;) {
    if (k == A.n - 1) {
      if (!emit(rest, A.stride[k] * r)) return TLA_ERR_UNSUPPORTED;
      return TLA_OK;
    }
    const int64_t steps = A.shape[k] / r;  // positions left in mode k
    if (rest <= steps) {
      if (!emit(rest, A.stride[k] * r)) return TLA_ERR_UNSUPPORTED;
      return TLA_OK;
    }
    if (rest % steps != 0) return TLA_ERR_UNSUPPORTED;
    if (!emit(steps, A.stride[k] * r)) return TLA_ERR_UNSUPPORTED;
    rest /= steps;
    r = 1;
    ++k;
  }
}

// The leaves of B must occupy disjoint digit ranges of A's mixed radix:
// sorted by stride, each leaf's range [d, d*s) ends at or before the next
// one's start.  Then A(sum of the leaves' indices) is the sum of A applied
// to each, which is what composing leaf by leaf assumes.
bool disjoint_digits(const Leaves& B) {
  int64_t d[TLA_MAX_LEAVES], s[TLA_MAX_LEAVES];
  int n = 0;
  for (int i = 0; i < B.n; ++i) {
    if (B.shape[i] == 1 || B.stride[i] == 0) continue;
    d[n] = B.stride[i];
    s[n] = B.shape[i];
    ++n;
  }
  int order[TLA_MAX_LEAVES];
  for (int i = 0; i < n; ++i) order[i] = i;
  std::sort(order, order + n, [&](int x, int y) { return d[x] < d[y]; });
  for (int i = 0; i + 1 < n; ++i) {
    const int a = order[i], b = order[i + 1];
    if (d[a] > d[b] / s[a]) return false;  // d[a]*s[a] > d[b], overflow-free
  }
  return true;
}

// Closed-form A o B keeping B's top-level modes.
int compose(const tla_layout* A, const tla_layout* B, tla_layout* out) {
  Leaves fa, fb, ca;
  int64_t sa, sb;
  int rc = read(A, &fa, &sa);
  if (rc) return rc;
  rc = read(B, &fb, &sb);
  if (rc) return rc;
  int64_t lo, hi;
  if (!value_range(fb, &lo, &hi) || lo < 0 || hi >= sa) return TLA_ERR_INVALID_ARG;
  coalesce_leaves(fa, &ca);
  if (!disjoint_digits(fb)) return TLA_ERR_UNSUPPORTED;
  tla_layout r;
  memset(&r, 0, sizeof(r));
  r.n_modes = B->n_modes;
  Leaves acc;
  int first[TLA_MAX_MODES];
  mode_starts(B, first);
  for (int m = 0; m < B->n_modes; ++m) {
    const int before = acc.n;
    for (int l = first[m]; l < first[m] + B->leaves[m]; ++l) {
      rc = compose_leaf(ca, fb.shape[l], fb.stride[l], &acc);
      if (rc) return rc;
    }
    r.leaves[m] = acc.n - before;
  }
  for (int i = 0; i < acc.n; ++i) {
    r.shape[i] = acc.shape[i];
    r.stride[i] = acc.stride[i];
  }
  *out = r;
  return TLA_OK;
}

// Mode m of L as a layout of its own (one mode, its leaves).
tla_layout mode_of(const tla_layout* L, int m) {
  int first[TLA_MAX_MODES];
  mode_starts(L, first);
  tla_layout r;
  memset(&r, 0, sizeof(r));
  r.n_modes = 1;
  r.leaves[0] = L->leaves[m];
  for (int i = 0; i < L->leaves[m]; ++i) {
    r.shape[i] = L->shape[first[m] + i];
    r.stride[i] = L->stride[first[m] + i];
  }
  return r;
}

}  // namespace

extern "C" {

int tla_logical_product(const tla_layout* L, const tla_layout* M, tla_layout* out) {
  Leaves fl, fm;
  int64_t sl, sm;
  int rc = read(L, &fl, &sl);
  if (rc) return rc;
  rc = read(M, &fm, &sm);
  if (rc) return rc;
  if (!out || L->n_modes + M->n_modes > TLA_MAX_MODES || fl.n + fm.n > TLA_MAX_LEAVES ||
      sl > INT64_MAX / sm)
    return TLA_ERR_INVALID_ARG;
  tla_layout r;
  memset(&r, 0, sizeof(r));
  r.n_modes = L->n_modes + M->n_modes;
  for (int i = 0; i < L->n_modes; ++i) r.leaves[i] = L->leaves[i];
  for (int i = 0; i < M->n_modes; ++i) r.leaves[L->n_modes + i] = M->leaves[i];
  for (int i = 0; i < fl.n; ++i) {
    r.shape[i] = fl.shape[i];
    r.stride[i] = fl.stride[i];
  }
  for (int i = 0; i < fm.n; ++i) {
    r.shape[fl.n + i] = fm.shape[i];
    r.stride[fl.n + i] = fm.stride[i];
  }
  *out = r;
  return TLA_OK;
}

int tla_coalesce(const tla_layout* L, tla_layout* out) {
  Leaves f, c;
  int64_t size;
  int rc = read(L, &f, &size);
  if (rc) return rc;
  if (!out) return TLA_ERR_INVALID_ARG;
  coalesce_leaves(f, &c);
  tla_layout r;
  memset(&r, 0, sizeof(r));
  r.n_modes = c.n;  // at most 16 leaves merge into at most 16 modes...
  if (r.n_modes > TLA_MAX_MODES) {
    // ...but a flat descriptor holds 8 modes: keep the leaves, nested in one mode
    r.n_modes = 1;
    r.leaves[0] = c.n;
  } else {
    for (int i = 0; i < c.n; ++i) r.leaves[i] = 1;
  }
  for (int i = 0; i < c.n; ++i) {
    r.shape[i] = c.shape[i];
    r.stride[i] = c.stride[i];
  }
  *out = r;
  return TLA_OK;
}

int tla_composition(const tla_layout* A, const tla_layout* B, tla_layout* out) {
  if (!out) return TLA_ERR_INVALID_ARG;
  return compose(A, B, out);
}

int tla_logical_divide_modes(const tla_layout* L, const int64_t* tile, int32_t n_tile,
                             tla_layout* out) {
  Leaves f;
  int64_t size;
  int rc = read(L, &f, &size);
  if (rc) return rc;
  if (!tile || !out || n_tile != L->n_modes || 2 * L->n_modes > TLA_MAX_MODES)
    return TLA_ERR_INVALID_ARG;
  for (int i = 0; i < n_tile; ++i)
    if (tile[i] < 1) return TLA_ERR_INVALID_ARG;
  tla_layout r;
  memset(&r, 0, sizeof(r));
  r.n_modes = 2 * L->n_modes;
  int used = 0;
  auto put = [&](int mode, const int64_t* shape, const int64_t* stride, int n) {
    if (used + n > TLA_MAX_LEAVES) return false;
    r.leaves[mode] = n;
    for (int i = 0; i < n; ++i) {
      r.shape[used + i] = shape[i];
      r.stride[used + i] = stride[i];
    }
    used += n;
    return true;
  };
  for (int m = 0; m < L->n_modes; ++m) {
    const tla_layout mode = mode_of(L, m);
    const int64_t t = tile[m];
    if (mode.leaves[0] == 1) {
      // one leaf n:d -> (t:d, ceil(n/t):d*t); ragged tiles allowed
      const int64_t n = mode.shape[0], d = mode.stride[0];
      const int64_t rest = (n + t - 1) / t;
      if (t > 1 && (d > INT64_MAX / t || d < INT64_MIN / t)) return TLA_ERR_INVALID_ARG;
      const int64_t s0[1] = {t}, d0[1] = {d}, s1[1] = {rest}, d1[1] = {d * t};
      if (!put(2 * m, s0, d0, 1) || !put(2 * m + 1, s1, d1, 1)) return TLA_ERR_UNSUPPORTED;
      continue;
    }
    int64_t n = 1;
    for (int i = 0; i < mode.leaves[0]; ++i) n *= mode.shape[i];
    if (n % t != 0) return TLA_ERR_UNSUPPORTED;
    tla_layout tiler, c;
    memset(&tiler, 0, sizeof(tiler));
    tiler.n_modes = 2;
    tiler.leaves[0] = tiler.leaves[1] = 1;
    tiler.shape[0] = t;
    tiler.stride[0] = 1;
    tiler.shape[1] = n / t;
    tiler.stride[1] = t;
    rc = compose(&mode, &tiler, &c);
    if (rc) return rc;
    if (!put(2 * m, c.shape, c.stride, c.leaves[0]) ||
        !put(2 * m + 1, c.shape + c.leaves[0], c.stride + c.leaves[0], c.leaves[1]))
      return TLA_ERR_UNSUPPORTED;
  }
  *out = r;
  return TLA_OK;
}

}  // extern "C"
