// api.cpp -- the C ABI of libtla.so: argument validation, status codes and
// dispatch to the HIP kernels.  Declarations and the contract of every entry
// point are in include/tla.h.
#include <string.h>

#include "kernels.hpp"
#include "tla/copy.hpp"
#include "tla/layout.hpp"

using namespace tla;

namespace {

bool valid_order(int o) { return o == TLA_ROW_MAJOR || o == TLA_COL_MAJOR; }
bool is_operand_type(int t) { return t == TLA_F16 || t == TLA_BF16 || t == TLA_E4M3; }
bool is_out_type(int t) { return t == TLA_F16 || t == TLA_BF16; }
bool is_aux_type(int t) { return t == TLA_F16 || t == TLA_BF16 || t == TLA_F32; }

int64_t max1(int64_t x) { return x > 1 ? x : 1; }

// Leading dimension needed by a rows x cols matrix in the given order.
int64_t min_ld(int order, int64_t rows, int64_t cols) {
  return max1(order == TLA_ROW_MAJOR ? cols : rows);
}

int validate_gemm(const tla_gemm_args* a, GemmProblem* p) {
  if (!a) return TLA_ERR_INVALID_ARG;
  if (a->M < 0 || a->N < 0 || a->K < 0) return TLA_ERR_INVALID_ARG;
  if (!valid_order(a->a_order) || !valid_order(a->b_order) || !valid_order(a->d_order))
    return TLA_ERR_INVALID_ARG;
  if (a->act < TLA_ACT_NONE || a->act > TLA_ACT_GELU) return TLA_ERR_INVALID_ARG;
  if (!is_operand_type(a->a_type) || a->b_type != a->a_type) return TLA_ERR_UNSUPPORTED;
  if (!is_out_type(a->d_type)) return TLA_ERR_UNSUPPORTED;
  const bool use_c = a->beta != 0.0f;
  if (use_c) {
    if (!a->C) return TLA_ERR_INVALID_ARG;
    if (!valid_order(a->c_order)) return TLA_ERR_INVALID_ARG;
    if (!is_aux_type(a->c_type)) return TLA_ERR_UNSUPPORTED;
  }
  if (a->bias && !is_aux_type(a->bias_type)) return TLA_ERR_UNSUPPORTED;
  if (a->M == 0 || a->N == 0) return 1;  // valid no-op
  if (!a->D) return TLA_ERR_INVALID_ARG;
  if (a->K > 0 && (!a->A || !a->B)) return TLA_ERR_INVALID_ARG;
  if (a->K > 0 && a->lda < min_ld(a->a_order, a->M, a->K)) return TLA_ERR_INVALID_ARG;
  if (a->K > 0 && a->ldb < min_ld(a->b_order, a->K, a->N)) return TLA_ERR_INVALID_ARG;
  if (a->ldd < min_ld(a->d_order, a->M, a->N)) return TLA_ERR_INVALID_ARG;
  if (use_c && a->ldc < min_ld(a->c_order, a->M, a->N)) return TLA_ERR_INVALID_ARG;
  // D may alias C only element for element
  if (use_c && a->C == a->D &&
      (a->c_order != a->d_order || a->ldc != a->ldd || a->c_type != a->d_type))
    return TLA_ERR_INVALID_ARG;
  p->M = a->M; p->N = a->N; p->K = a->K;
  p->A = a->A; p->a_type = a->a_type; p->a_order = a->a_order; p->lda = a->lda;
  p->B = a->B; p->b_type = a->b_type; p->b_order = a->b_order; p->ldb = a->ldb;
  p->C = use_c ? a->C : nullptr; p->c_type = use_c ? a->c_type : a->d_type;
  p->c_order = use_c ? a->c_order : TLA_ROW_MAJOR; p->ldc = use_c ? a->ldc : 0;
  p->D = a->D; p->d_type = a->d_type; p->d_order = a->d_order; p->ldd = a->ldd;
  p->bias = a->bias; p->bias_type = a->bias ? a->bias_type : TLA_F32;
  p->act = a->act;
  p->alpha_eff = a->alpha * a->scale_a * a->scale_b;
  p->beta = use_c ? a->beta : 0.0f;
  return TLA_OK;
}

// Flattened leaves of a descriptor after its structural checks; size via
// overflow-checked product.
int flatten(const tla_layout* L, FlatLayout* f, int64_t* size) {
  if (!L || L->n_modes < 1 || L->n_modes > TLA_MAX_MODES) return TLA_ERR_INVALID_ARG;
  int n = 0;
  for (int i = 0; i < L->n_modes; ++i) {
    if (L->leaves[i] < 1) return TLA_ERR_INVALID_ARG;
    n += L->leaves[i];
  }
  if (n > TLA_MAX_LEAVES) return TLA_ERR_INVALID_ARG;
  int64_t s = 1;
  f->n = n;
  for (int i = 0; i < n; ++i) {
    if (L->shape[i] < 1) return TLA_ERR_INVALID_ARG;
    if (s > INT64_MAX / L->shape[i]) return TLA_ERR_INVALID_ARG;
    s *= L->shape[i];
    f->shape[i] = L->shape[i];
    f->stride[i] = L->stride[i];
  }
  if (size) *size = s;
  return TLA_OK;
}

bool is_flat(const tla_layout* L) {
  for (int i = 0; i < L->n_modes; ++i)
    if (L->leaves[i] != 1) return false;
  return true;
}

// Range [lo, hi] of a flat layout's values (each leaf contributes from 0 to
// (extent-1)*stride, so the extremes are sums of per-leaf extremes).
void value_range(const FlatLayout& f, int64_t* lo, int64_t* hi) {
  int64_t a = 0, b = 0;
  for (int i = 0; i < f.n; ++i) {
    const int64_t span = (f.shape[i] - 1) * f.stride[i];
    if (span < 0) a += span; else b += span;
  }
  *lo = a; *hi = b;
}

template <int R>
void divide_fixed(const tla_layout* L, const int64_t* tile, bool tiled, tla_layout* out) {
  Layout<R, int64_t> in{};
  int64_t t[R];
  for (int i = 0; i < R; ++i) {
    in.shape[i] = L->shape[i];
    in.stride[i] = L->stride[i];
    t[i] = tile[i];
  }
  const Layout<2 * R, int64_t> d = tiled ? tiled_divide(in, t) : logical_divide(in, t);
  memset(out, 0, sizeof(*out));
  if (tiled) {
    out->n_modes = 1 + R;
    out->leaves[0] = R;
    for (int i = 1; i <= R; ++i) out->leaves[i] = 1;
  } else {
    out->n_modes = R;
    for (int i = 0; i < R; ++i) out->leaves[i] = 2;
  }
  for (int i = 0; i < 2 * R; ++i) {
    out->shape[i] = d.shape[i];
    out->stride[i] = d.stride[i];
  }
}

int divide(const tla_layout* L, const int64_t* tile, int32_t n_tile, tla_layout* out, bool tiled) {
  FlatLayout f;
  int64_t size;
  int rc = flatten(L, &f, &size);
  if (rc) return rc;
  if (!tile || !out || !is_flat(L) || n_tile != L->n_modes) return TLA_ERR_INVALID_ARG;
  if (tiled && L->n_modes > TLA_MAX_MODES - 1) return TLA_ERR_INVALID_ARG;
  for (int i = 0; i < n_tile; ++i)
    if (tile[i] < 1) return TLA_ERR_INVALID_ARG;
  switch (n_tile) {
    case 1: divide_fixed<1>(L, tile, tiled, out); break;
    case 2: divide_fixed<2>(L, tile, tiled, out); break;
    case 3: divide_fixed<3>(L, tile, tiled, out); break;
    case 4: divide_fixed<4>(L, tile, tiled, out); break;
    case 5: divide_fixed<5>(L, tile, tiled, out); break;
    case 6: divide_fixed<6>(L, tile, tiled, out); break;
    case 7: divide_fixed<7>(L, tile, tiled, out); break;
    case 8: divide_fixed<8>(L, tile, tiled, out); break;
    default: return TLA_ERR_INVALID_ARG;
  }
  return TLA_OK;
}

int check_thread_map(int64_t R, int64_t C, int32_t T, int32_t V, int32_t I, int32_t contig,
                     int32_t threads_per_row = 0, int32_t swizzle_shift = -1) {
  if (R < 1 || C < 1 || T < 1 || V < 1 || I < 1) return TLA_ERR_INVALID_ARG;
  if (contig != 0 && contig != 1) return TLA_ERR_INVALID_ARG;
  if (threads_per_row < 0 || swizzle_shift < -1) return TLA_ERR_INVALID_ARG;
  if (R > (1 << 20) || C > (1 << 20) || R * C > (int64_t(1) << 28)) return TLA_ERR_INVALID_ARG;
  const StripMinedMap map((int)R, (int)C, T, V, I, contig, threads_per_row, swizzle_shift);
  return map.well_formed() ? TLA_OK : TLA_ERR_INVALID_ARG;
}

int validate_conv(const tla_conv2d_args* a, ConvProblem* out) {
  if (!a) return TLA_ERR_INVALID_ARG;
  if (a->N < 0 || a->H < 1 || a->W < 1 || a->C < 1 || a->K < 1 || a->R < 1 || a->S < 1)
    return TLA_ERR_INVALID_ARG;
  if (a->stride_h < 1 || a->stride_w < 1 || a->dil_h < 1 || a->dil_w < 1 || a->pad_h < 0 ||
      a->pad_w < 0 || a->act < TLA_ACT_NONE || a->act > TLA_ACT_GELU)
    return TLA_ERR_INVALID_ARG;
  if (!is_out_type(a->type)) return TLA_ERR_UNSUPPORTED;
  if (a->bias && !is_aux_type(a->bias_type)) return TLA_ERR_UNSUPPORTED;
  const int64_t lim = int64_t(1) << 31;
  if (a->H > lim || a->W > lim || a->R > lim || a->S > lim) return TLA_ERR_INVALID_ARG;
  // padded extents below 2^30 keep every image coordinate the kernels form
  // (p*u - ph + r*dh and the like) inside a 32-bit int
  if (a->H + 2 * (int64_t)a->pad_h >= (lim >> 1) || a->W + 2 * (int64_t)a->pad_w >= (lim >> 1))
    return TLA_ERR_INVALID_ARG;
  const int64_t ph = a->H + 2 * (int64_t)a->pad_h - (int64_t)a->dil_h * (a->R - 1) - 1;
  const int64_t pw = a->W + 2 * (int64_t)a->pad_w - (int64_t)a->dil_w * (a->S - 1) - 1;
  const int64_t P = ph < 0 ? 0 : ph / a->stride_h + 1, Q = pw < 0 ? 0 : pw / a->stride_w + 1;
  if (a->N == 0 || P < 1 || Q < 1) return 1;  // nothing to do
  if (!a->x || !a->w || !a->y) return TLA_ERR_INVALID_ARG;
  if (a->beta != 0.0f && !a->C_res) return TLA_ERR_INVALID_ARG;
  if (a->N > lim / P || a->N * P > lim / Q || a->K >= lim || a->C > lim / (a->R * a->S) ||
      a->R * a->S > lim || a->N * a->H > lim / a->W || a->N * a->H * a->W > lim / a->C)
    return TLA_ERR_INVALID_ARG;
  if (a->N * P * Q >= lim || a->R * a->S * a->C >= lim) return TLA_ERR_INVALID_ARG;
  ConvProblem& c = *out;
  c = ConvProblem{};
  c.N = a->N; c.H = a->H; c.W = a->W; c.C_in = a->C; c.K = a->K; c.R = a->R; c.S = a->S;
  c.P = P; c.Q = Q;
  c.u = a->stride_h; c.v = a->stride_w; c.ph = a->pad_h; c.pw = a->pad_w;
  c.dh = a->dil_h; c.dw = a->dil_w;
  c.x = a->x; c.w = a->w; c.C = a->beta != 0.0f ? a->C_res : nullptr; c.y = a->y;
  c.type = a->type; c.bias = a->bias; c.bias_type = a->bias ? a->bias_type : TLA_F32;
  c.act = a->act; c.alpha = a->alpha; c.beta = a->beta;
  return TLA_OK;
}

}  // namespace

extern "C" {

int tla_gemm_epilogue(const tla_gemm_args* args, void* stream) {
  GemmProblem p{};
  const int rc = validate_gemm(args, &p);
  if (rc < 0) return rc;
  if (rc == 1) return TLA_OK;
  return gemm_dispatch(p, (hipStream_t)stream, false, nullptr);
}

int tla_conv2d_fprop(const tla_conv2d_args* a, void* stream) {
  ConvProblem c;
  const int rc = validate_conv(a, &c);
  if (rc < 0) return rc;
  if (rc == 1) return TLA_OK;
  return conv_dispatch(c, (hipStream_t)stream);
}

int tla_conv2d_fprop_variant(const tla_conv2d_args* a, int32_t variant, void* stream) {
  if (variant < 0 || variant >= TLA_CONV_VARIANTS) return TLA_ERR_INVALID_ARG;
  ConvProblem c;
  const int rc = validate_conv(a, &c);
  if (rc < 0) return rc;
  if (rc == 1) return TLA_OK;
  return conv_dispatch(c, (hipStream_t)stream, variant);
}

int tla_gemm_run_variant(const tla_gemm_args* args, int32_t variant, void* stream) {
  if (variant < 0 || variant >= kGemmVariants) return TLA_ERR_INVALID_ARG;
  GemmProblem p{};
  const int rc = validate_gemm(args, &p);
  if (rc < 0) return rc;
  if (rc == 1) return TLA_OK;
  return gemm_dispatch(p, (hipStream_t)stream, false, nullptr, variant);
}

int tla_gemm_variant_info(int32_t variant, int32_t a_type, tla_gemm_kernel_info* out) {
  if (!out || variant < 0 || variant >= kGemmVariants) return TLA_ERR_INVALID_ARG;
  GemmKernelInfo k{};
  const int rc = gemm_variant_info(a_type, variant, &k);
  if (rc) return rc;
  memset(out, 0, sizeof(*out));
  strncpy(out->name, k.name, sizeof(out->name) - 1);
  out->block_m = out->block_n = k.tile;
  out->threads = k.threads;
  out->lds_bytes = k.lds_bytes;
  out->vgprs = k.vgprs;
  out->blocks_per_cu = k.blocks_per_cu;
  return TLA_OK;
}

int tla_gemm_variant(const tla_gemm_args* args, char* buf, int32_t cap) {
  if (!buf || cap < 1) return TLA_ERR_INVALID_ARG;
  GemmProblem p{};
  const int rc = validate_gemm(args, &p);
  if (rc < 0) return rc;
  const char* name = "noop";
  if (rc == 0) {
    const int r2 = gemm_dispatch(p, nullptr, true, &name);
    if (r2) return r2;
  }
  strncpy(buf, name, (size_t)cap - 1);
  buf[cap - 1] = '\0';
  return TLA_OK;
}

int tla_tiled_transpose(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t M,
                        int64_t N, int32_t elem_bytes, void* stream) {
  if (M < 0 || N < 0) return TLA_ERR_INVALID_ARG;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8 && elem_bytes != 16)
    return TLA_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return TLA_OK;
  if (!src || !dst || ld_src < N || ld_dst < M) return TLA_ERR_INVALID_ARG;
  if (((uintptr_t)src % (uintptr_t)elem_bytes) || ((uintptr_t)dst % (uintptr_t)elem_bytes))
    return TLA_ERR_INVALID_ARG;
  const uintptr_t s0 = (uintptr_t)src, s1 = s0 + (uintptr_t)(((M - 1) * ld_src + N) * elem_bytes);
  const uintptr_t d0 = (uintptr_t)dst, d1 = d0 + (uintptr_t)(((N - 1) * ld_dst + M) * elem_bytes);
  if (s0 < d1 && d0 < s1) return TLA_ERR_OVERLAP;
  return transpose_dispatch(src, ld_src, dst, ld_dst, M, N, elem_bytes, (hipStream_t)stream);
}

int tla_tiled_copy(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t M,
                   int64_t N, int32_t elem_bytes, void* stream) {
  if (M < 0 || N < 0) return TLA_ERR_INVALID_ARG;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8 && elem_bytes != 16)
    return TLA_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return TLA_OK;
  if (!src || !dst || ld_src < N || ld_dst < N) return TLA_ERR_INVALID_ARG;
  if (((uintptr_t)src % (uintptr_t)elem_bytes) || ((uintptr_t)dst % (uintptr_t)elem_bytes))
    return TLA_ERR_INVALID_ARG;
  const uintptr_t s0 = (uintptr_t)src, s1 = s0 + (uintptr_t)(((M - 1) * ld_src + N) * elem_bytes);
  const uintptr_t d0 = (uintptr_t)dst, d1 = d0 + (uintptr_t)(((M - 1) * ld_dst + N) * elem_bytes);
  if (s0 < d1 && d0 < s1) return TLA_ERR_OVERLAP;
  return copy_dispatch(src, ld_src, dst, ld_dst, M, N, elem_bytes, (hipStream_t)stream);
}

int tla_layout_size(const tla_layout* L, int64_t* size) {
  if (!size) return TLA_ERR_INVALID_ARG;
  FlatLayout f;
  return flatten(L, &f, size);
}

int tla_layout_eval(const tla_layout* outer, const tla_layout* inner, int64_t* out, int64_t n,
                    void* stream) {
  FlatLayout fo{}, fi{};
  int64_t so = 0, si = 0;
  int rc = flatten(outer, &fo, &so);
  if (rc) return rc;
  if (inner) {
    rc = flatten(inner, &fi, &si);
    if (rc) return rc;
    if (n != si) return TLA_ERR_INVALID_ARG;
    int64_t lo, hi;
    value_range(fi, &lo, &hi);
    if (lo < 0 || hi >= so) return TLA_ERR_INVALID_ARG;
  } else if (n != so) {
    return TLA_ERR_INVALID_ARG;
  }
  if (n > 0 && !out) return TLA_ERR_INVALID_ARG;
  return layout_eval_dispatch(fo, fi, inner != nullptr, out, n, (hipStream_t)stream);
}

int tla_logical_divide(const tla_layout* L, const int64_t* tile, int32_t n_tile, tla_layout* out) {
  return divide(L, tile, n_tile, out, false);
}

int tla_tiled_divide(const tla_layout* L, const int64_t* tile, int32_t n_tile, tla_layout* out) {
  return divide(L, tile, n_tile, out, true);
}

int tla_thread_map_ex(int64_t R, int64_t C, int32_t T, int32_t V, int32_t I,
                      int32_t contiguous_dim, int32_t threads_per_row, tla_layout* out) {
  if (!out) return TLA_ERR_INVALID_ARG;
  const int rc = check_thread_map(R, C, T, V, I, contiguous_dim, threads_per_row);
  if (rc) return rc;
  const StripMinedMap map((int)R, (int)C, T, V, I, contiguous_dim, threads_per_row);
  memset(out, 0, sizeof(*out));
  out->n_modes = 2;
  out->leaves[0] = 2;
  if (map.Ic == 1) {
    const Layout<4, int> tv = map.tv_layout();
    out->leaves[1] = 2;
    for (int i = 0; i < 4; ++i) {
      out->shape[i] = tv.shape[i];
      out->stride[i] = tv.stride[i];
    }
  } else {
    // ((G, T/G), (V, Ic, I/Ic)) : ((V, Q), (1, G*V, S*Q))
    out->leaves[1] = 3;
    const int64_t shape[5] = {map.G, map.T / map.G, map.V, map.Ic, map.I / map.Ic};
    const int64_t stride[5] = {map.V, map.Q, 1, (int64_t)map.G * map.V, (int64_t)map.S * map.Q};
    for (int i = 0; i < 5; ++i) {
      out->shape[i] = shape[i];
      out->stride[i] = stride[i];
    }
  }
  return TLA_OK;
}

int tla_thread_map(int64_t R, int64_t C, int32_t T, int32_t V, int32_t I, int32_t contiguous_dim,
                   tla_layout* out) {
  return tla_thread_map_ex(R, C, T, V, I, contiguous_dim, 0, out);
}

int tla_thread_map_eval_ex(int64_t R, int64_t C, int32_t T, int32_t V, int32_t I,
                           int32_t contiguous_dim, int32_t threads_per_row, int32_t swizzle_shift,
                           int64_t rows_valid, int64_t cols_valid, int64_t* out_index,
                           uint8_t* out_valid, void* stream) {
  const int rc = check_thread_map(R, C, T, V, I, contiguous_dim, threads_per_row, swizzle_shift);
  if (rc) return rc;
  if (!out_index || rows_valid < 0 || cols_valid < 0) return TLA_ERR_INVALID_ARG;
  return thread_map_eval_dispatch((int)R, (int)C, T, V, I, contiguous_dim, threads_per_row,
                                  swizzle_shift, rows_valid, cols_valid, out_index, out_valid,
                                  (hipStream_t)stream);
}

int tla_thread_map_eval(int64_t R, int64_t C, int32_t T, int32_t V, int32_t I,
                        int32_t contiguous_dim, int64_t rows_valid, int64_t cols_valid,
                        int64_t* out_index, uint8_t* out_valid, void* stream) {
  return tla_thread_map_eval_ex(R, C, T, V, I, contiguous_dim, 0, -1, rows_valid, cols_valid,
                                out_index, out_valid, stream);
}

const char* tla_status_string(int status) {
  switch (status) {
    case TLA_OK: return "TLA_OK";
    case TLA_ERR_INVALID_ARG: return "TLA_ERR_INVALID_ARG";
    case TLA_ERR_UNSUPPORTED: return "TLA_ERR_UNSUPPORTED";
    case TLA_ERR_OVERLAP: return "TLA_ERR_OVERLAP";
    case TLA_ERR_HIP: return "TLA_ERR_HIP";
    default: return "TLA_ERR_UNKNOWN";
  }
}

int tla_version(void) { return 1; }

}  // extern "C"
