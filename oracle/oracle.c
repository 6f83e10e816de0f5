/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the tiled GEMM
 * with fused epilogue and for the row-major -> column-major transpose.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include,
 * link or call this file.  Only the test-suite, the smoke check and the
 * bench's cpu_baseline leg use it.  It shares no code, header or constant
 * table with the HIP library: every decoder, index map and epilogue step
 * below is written out independently from its textbook definition.
 *
 * What it computes (all in IEEE binary64, no output rounding):
 *
 *   ref(m,n) = act( alpha*scale_a*scale_b * sum_{k<K} A(m,k)*B(k,n)
 *                   + beta*C(m,n)      (only when beta != 0)
 *                   + bias(n) )        (only when bias != NULL)
 *
 *   - the GEMM problem statement C[M,N] = A[M,K] x B[K,N] and its mapping to
 *     the block/warp/instruction hierarchy: "CUTLASS / CuTe 主线"
 *     (hpc.payai.win/cutlass), section 一 "先把 GEMM 三重循环映射到 GPU 层级";
 *   - the epilogue (alpha/beta, bias/activation, store): same page, section 一
 *     box "Epilogue" and section 三 box "Collective Epilogue";
 *   - mixed precision with an fp32 accumulator: same page, lesson 7 in the
 *     course table.  The oracle accumulates in fp64, a superset of fp32.
 *   - the naive triple loop is the first step of that page's exercise path
 *     (section 四, "练习路线": naive GEMM -> tiled GEMM -> ...).
 *
 * Operand views: an operand element (r,c) lives at index
 *   crd2idx((r,c), stride) = r*stride_r + c*stride_c
 * with stride (ld,1) for row-major and (1,ld) for column-major storage: the
 * Layout = (Shape, Stride) dot-product rule of "Advanced CUTLASS Architecture
 * and Kernel Optimization" (oboe.com), section "The Algebra of Layouts", with
 * the pitch taken from the tensor layout as in the PitchLinearStripminedThreadMap
 * walk-through (lpnh.cn), section 6.3.
 *
 * Summation is a single dependent chain over k = 0..K-1 in binary64.  Host
 * threads split the output rows; each (m,n) is still summed by one thread in
 * the same order, so the result does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* storage type codes (same numbering as the public C header, written out
 * here again on purpose: the oracle includes nothing from the library) */
enum { OR_F16 = 0, OR_BF16 = 1, OR_E4M3 = 2, OR_F32 = 3 };
enum { OR_ROW = 0, OR_COL = 1 };
enum { OR_ACT_NONE = 0, OR_ACT_RELU = 1, OR_ACT_GELU = 2 };

/* ---------------------------------------------------------------- decoders */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double dec_f16(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-14 / 2^10 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(1024.0 + f, e - 25); /* (1 + f/2^10) * 2^(e-15) */
  return s ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double dec_bf16(uint16_t b) {
  int s = (b >> 15) & 1, e = (b >> 7) & 255, f = b & 127;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133); /* f * 2^-126 / 2^7 */
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(128.0 + f, e - 134); /* (1 + f/2^7) * 2^(e-127) */
  return s ? -v : v;
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; largest finite 0x7E = 448. */
static double dec_e4m3(uint8_t x) {
  int s = (x >> 7) & 1, e = (x >> 3) & 15, f = x & 7;
  double v;
  if (e == 15 && f == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)f, -9); /* f * 2^-6 / 2^3 */
  else
    v = ldexp(8.0 + f, e - 10); /* (1 + f/8) * 2^(e-7) */
  return s ? -v : v;
}

/* IEEE 754 binary32, decoded from its fields (not by a type pun). */
static double dec_f32(uint32_t u) {
  int s = (u >> 31) & 1, e = (u >> 23) & 255;
  uint32_t f = u & 0x7FFFFFu;
  double v;
  if (e == 0)
    v = ldexp((double)f, -149);
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(8388608.0 + f, e - 150);
  return s ? -v : v;
}

static int elem_bytes(int t) {
  switch (t) {
  case OR_F16: case OR_BF16: return 2;
  case OR_E4M3: return 1;
  case OR_F32: return 4;
  default: return 0;
  }
}

static double decode_at(int t, const void *base, int64_t i) {
  switch (t) {
  case OR_F16: { uint16_t h; memcpy(&h, (const char *)base + 2 * i, 2); return dec_f16(h); }
  case OR_BF16: { uint16_t h; memcpy(&h, (const char *)base + 2 * i, 2); return dec_bf16(h); }
  case OR_E4M3: return dec_e4m3(((const uint8_t *)base)[i]);
  case OR_F32: { uint32_t u; memcpy(&u, (const char *)base + 4 * i, 4); return dec_f32(u); }
  default: return NAN;
  }
}

/* Decode n consecutive elements of storage type t into binary64. */
int oracle_decode(int t, const void *src, int64_t n, double *out) {
  if (!elem_bytes(t) || n < 0 || (n && (!src || !out))) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = decode_at(t, src, i);
  return 0;
}

/* ------------------------------------------------------------ operand view */

/* crd2idx of a 2-D coordinate under a (Shape, Stride) layout whose strides
 * are (ld,1) (row-major) or (1,ld) (column-major). */
static int64_t crd2idx2(int64_t r, int64_t c, int order, int64_t ld) {
  int64_t s_r = (order == OR_ROW) ? ld : 1;
  int64_t s_c = (order == OR_ROW) ? 1 : ld;
  return r * s_r + c * s_c;
}

typedef struct {
  int64_t M, N, K;
  const void *A; int32_t a_type, a_order; int64_t lda;
  const void *B; int32_t b_type, b_order; int64_t ldb;
  const void *C; int32_t c_type, c_order; int64_t ldc;
  const void *bias; int32_t bias_type; int32_t act;
  double alpha, beta, scale_a, scale_b;
} oracle_gemm_args;

/* Gaussian error linear unit, exact erf form: y * Phi(y). */
static double gelu(double y) { return 0.5 * y * (1.0 + erf(y / sqrt(2.0))); }

static double epilogue(const oracle_gemm_args *a, double s, int64_t m, int64_t n) {
  double y = a->alpha * a->scale_a * a->scale_b * s;
  if (a->beta != 0.0)
    y += a->beta * decode_at(a->c_type, a->C, crd2idx2(m, n, a->c_order, a->ldc));
  if (a->bias) y += decode_at(a->bias_type, a->bias, n);
  if (a->act == OR_ACT_RELU) y = (y > 0.0) ? y : 0.0;
  else if (a->act == OR_ACT_GELU) y = gelu(y);
  return y;
}

static int check_args(const oracle_gemm_args *a) {
  if (!a || a->M < 0 || a->N < 0 || a->K < 0) return -1;
  if (!elem_bytes(a->a_type) || !elem_bytes(a->b_type)) return -1;
  if (a->K > 0 && a->M > 0 && !a->A) return -1;
  if (a->K > 0 && a->N > 0 && !a->B) return -1;
  if (a->beta != 0.0 && (!a->C || !elem_bytes(a->c_type))) return -1;
  if (a->bias && !elem_bytes(a->bias_type)) return -1;
  return 0;
}

/* Full GEMM.  Operands are first normalised into binary64 A[M][K] and
 * B^T[N][K] (so the k-loop reads both contiguously); then the naive triple
 * loop. */
typedef struct {
  const oracle_gemm_args *a;
  const double *Ad, *Btd;
  double *ref;
  int64_t m0, m1;
} gemm_job;

static void *gemm_rows(void *p) {
  gemm_job *j = (gemm_job *)p;
  const oracle_gemm_args *a = j->a;
  for (int64_t m = j->m0; m < j->m1; ++m) {
    const double *ar = j->Ad + m * a->K;
    for (int64_t n = 0; n < a->N; ++n) {
      const double *br = j->Btd + n * a->K;
      double s = 0.0;
      for (int64_t k = 0; k < a->K; ++k) s += ar[k] * br[k];
      j->ref[m * a->N + n] = epilogue(a, s, m, n);
    }
  }
  return NULL;
}

typedef struct {
  const oracle_gemm_args *a;
  double *Ad, *Btd;
  int64_t r0, r1; /* rows of A first, then rows of B^T, as one index range */
} norm_job;

static void *normalise_rows(void *p) {
  norm_job *j = (norm_job *)p;
  const oracle_gemm_args *a = j->a;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    if (r < a->M) {
      for (int64_t k = 0; k < a->K; ++k)
        j->Ad[r * a->K + k] = decode_at(a->a_type, a->A, crd2idx2(r, k, a->a_order, a->lda));
    } else {
      int64_t n = r - a->M;
      for (int64_t k = 0; k < a->K; ++k)
        j->Btd[n * a->K + k] = decode_at(a->b_type, a->B, crd2idx2(k, n, a->b_order, a->ldb));
    }
  }
  return NULL;
}

int oracle_gemm(const oracle_gemm_args *a, double *ref, int nthreads) {
  if (check_args(a) || (a->M * a->N > 0 && !ref)) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (a->M == 0 || a->N == 0) return 0;
  double *Ad = (double *)malloc(sizeof(double) * (size_t)(a->M * a->K + 1));
  double *Btd = (double *)malloc(sizeof(double) * (size_t)(a->N * a->K + 1));
  if (!Ad || !Btd) { free(Ad); free(Btd); return -2; }
  pthread_t th[256];
  {
    norm_job jobs[256];
    int64_t rows = a->M + a->N;
    for (int t = 0; t < nthreads; ++t) {
      jobs[t].a = a; jobs[t].Ad = Ad; jobs[t].Btd = Btd;
      jobs[t].r0 = rows * t / nthreads; jobs[t].r1 = rows * (t + 1) / nthreads;
      pthread_create(&th[t], NULL, normalise_rows, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  }
  {
    gemm_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
      jobs[t].a = a; jobs[t].Ad = Ad; jobs[t].Btd = Btd; jobs[t].ref = ref;
      jobs[t].m0 = a->M * t / nthreads; jobs[t].m1 = a->M * (t + 1) / nthreads;
      pthread_create(&th[t], NULL, gemm_rows, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  }
  free(Ad); free(Btd);
  return 0;
}

/* Selected outputs only: out[i] = ref(ms[i], ns[i]), each summed directly
 * from the stored operands with the same sequential k-order as oracle_gemm. */
typedef struct {
  const oracle_gemm_args *a;
  const int64_t *ms, *ns;
  double *out;
  int64_t i0, i1;
} point_job;

static void *gemm_points_run(void *p) {
  point_job *j = (point_job *)p;
  const oracle_gemm_args *a = j->a;
  for (int64_t i = j->i0; i < j->i1; ++i) {
    int64_t m = j->ms[i], n = j->ns[i];
    double s = 0.0;
    for (int64_t k = 0; k < a->K; ++k)
      s += decode_at(a->a_type, a->A, crd2idx2(m, k, a->a_order, a->lda)) *
           decode_at(a->b_type, a->B, crd2idx2(k, n, a->b_order, a->ldb));
    j->out[i] = epilogue(a, s, m, n);
  }
  return NULL;
}

int oracle_gemm_points(const oracle_gemm_args *a, const int64_t *ms, const int64_t *ns,
                       int64_t count, double *out, int nthreads) {
  if (check_args(a) || count < 0 || (count && (!ms || !ns || !out))) return -1;
  for (int64_t i = 0; i < count; ++i)
    if (ms[i] < 0 || ms[i] >= a->M || ns[i] < 0 || ns[i] >= a->N) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  point_job jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].a = a; jobs[t].ms = ms; jobs[t].ns = ns; jobs[t].out = out;
    jobs[t].i0 = count * t / nthreads; jobs[t].i1 = count * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, gemm_points_run, &jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}

/* ------------------------------------------------------------- transpose */

/* Row-major S (M x N, pitch ld_src) -> column-major D (pitch ld_dst):
 * D(m,n) = S(m,n) bit for bit, i.e. dst[m + n*ld_dst] = src[m*ld_src + n].
 * Defined in "什么是 CuTe ?" (GPU Glossary zh, 4.21): the transpose kernel
 * copies a row-major tensor into a column-major one over the same shape. */
int oracle_transpose(const void *src, int64_t ld_src, void *dst, int64_t ld_dst,
                     int64_t M, int64_t N, int32_t eb) {
  if (M < 0 || N < 0 || eb <= 0) return -1;
  if (M == 0 || N == 0) return 0;
  if (!src || !dst || ld_src < N || ld_dst < M) return -1;
  const char *s = (const char *)src;
  char *d = (char *)dst;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n)
      memcpy(d + (m + n * ld_dst) * eb, s + (m * ld_src + n) * eb, (size_t)eb);
  return 0;
}

/* Row-major S (M x N, pitch ld_src) -> row-major D (pitch ld_dst): the
 * identity case of the same layout-driven copy, D(m,n) = S(m,n) bit for
 * bit, i.e. dst[m*ld_dst + n] = src[m*ld_src + n].  Padding of D is not
 * written. */
int oracle_copy2d(const void *src, int64_t ld_src, void *dst, int64_t ld_dst,
                  int64_t M, int64_t N, int32_t eb) {
  if (M < 0 || N < 0 || eb <= 0) return -1;
  if (M == 0 || N == 0) return 0;
  if (!src || !dst || ld_src < N || ld_dst < N) return -1;
  const char *s = (const char *)src;
  char *d = (char *)dst;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n)
      memcpy(d + (m * ld_dst + n) * eb, s + (m * ld_src + n) * eb, (size_t)eb);
  return 0;
}

/* ----------------------------------------------------------- convolution */

/* Forward convolution (cross-correlation) as the implicit GEMM of the
 * PitchLinearStripminedThreadMap walk-through (lpnh.cn/news/2469163),
 * section 5.2: one GEMM dimension is the output pixel, the other the
 * filter position times the channel.  Reading (the page gives no formula):
 * x is N x H x W x C (NHWC), w is K x R x S x C (KRSC), the output N x P x Q x K
 * (NPQK) with P = (H + 2 ph - dh (R-1) - 1) / u + 1 (Q likewise), and
 *   s[n,p,q,k] = sum over r < R, s < S, c < C of
 *                x[n, p u - ph + r dh, q v - pw + s dw, c] * w[k, r, s, c],
 * x taken as 0 outside the image.  The GEMM epilogue follows at GEMM
 * position (m = (n P + p) Q + q, k): alpha, beta * Cres[n,p,q,k], bias[k],
 * activation. */
typedef struct {
  int64_t N, H, W, C, K, R, S;
  int32_t u, v, ph, pw, dh, dw;
  const void *x; const void *w; const void *Cres; int32_t type;
  const void *bias; int32_t bias_type; int32_t act;
  double alpha, beta;
} oracle_conv_args;

static int64_t conv_out(int64_t in, int64_t f, int32_t stride, int32_t pad, int32_t dil) {
  const int64_t span = in + 2 * (int64_t)pad - (int64_t)dil * (f - 1) - 1;
  return span < 0 ? 0 : span / stride + 1;
}

typedef struct {
  const oracle_conv_args *a;
  const double *xd, *wd;
  oracle_gemm_args g;          /* the epilogue's view: M = NPQ, N = K */
  int64_t P, Q;
  const int64_t *ms, *ks;      /* points mode when non-NULL */
  double *out;
  int64_t i0, i1;              /* output rows (full) or points */
} conv_job;

static double conv_sum(const conv_job *j, int64_t m, int64_t k) {
  const oracle_conv_args *a = j->a;
  const int64_t q = m % j->Q, p = (m / j->Q) % j->P, n = m / (j->Q * j->P);
  double s = 0.0;
  for (int64_t r = 0; r < a->R; ++r) {
    const int64_t h = p * a->u - a->ph + r * a->dh;
    if (h < 0 || h >= a->H) continue;
    for (int64_t t = 0; t < a->S; ++t) {
      const int64_t w = q * a->v - a->pw + t * a->dw;
      if (w < 0 || w >= a->W) continue;
      const double *xr = j->xd + ((n * a->H + h) * a->W + w) * a->C;
      const double *wr = j->wd + ((k * a->R + r) * a->S + t) * a->C;
      for (int64_t c = 0; c < a->C; ++c) s += xr[c] * wr[c];
    }
  }
  return s;
}

static void *conv_run(void *p) {
  conv_job *j = (conv_job *)p;
  if (j->ms) {
    for (int64_t i = j->i0; i < j->i1; ++i)
      j->out[i] = epilogue(&j->g, conv_sum(j, j->ms[i], j->ks[i]), j->ms[i], j->ks[i]);
  } else {
    for (int64_t m = j->i0; m < j->i1; ++m)
      for (int64_t k = 0; k < j->a->K; ++k)
        j->out[m * j->a->K + k] = epilogue(&j->g, conv_sum(j, m, k), m, k);
  }
  return NULL;
}

static int conv_common(const oracle_conv_args *a, const int64_t *ms, const int64_t *ks,
                       int64_t npts, double *out, int nthreads) {
  if (!a || !out || a->N < 0 || a->H < 1 || a->W < 1 || a->C < 1 || a->K < 1 || a->R < 1 ||
      a->S < 1 || a->u < 1 || a->v < 1 || a->dh < 1 || a->dw < 1 || a->ph < 0 || a->pw < 0 ||
      !elem_bytes(a->type) || !a->x || !a->w)
    return -1;
  const int64_t P = conv_out(a->H, a->R, a->u, a->ph, a->dh);
  const int64_t Q = conv_out(a->W, a->S, a->v, a->pw, a->dw);
  const int64_t nx = a->N * a->H * a->W * a->C, nw = a->K * a->R * a->S * a->C;
  double *xd = (double *)malloc(sizeof(double) * (size_t)(nx > 0 ? nx : 1));
  double *wd = (double *)malloc(sizeof(double) * (size_t)nw);
  if (!xd || !wd) { free(xd); free(wd); return -2; }
  for (int64_t i = 0; i < nx; ++i) xd[i] = decode_at(a->type, a->x, i);
  for (int64_t i = 0; i < nw; ++i) wd[i] = decode_at(a->type, a->w, i);
  oracle_gemm_args g;
  memset(&g, 0, sizeof(g));
  g.M = a->N * P * Q; g.N = a->K; g.K = a->R * a->S * a->C;
  g.C = a->Cres; g.c_type = a->type; g.c_order = OR_ROW; g.ldc = a->K;
  g.bias = a->bias; g.bias_type = a->bias_type; g.act = a->act;
  g.alpha = a->alpha; g.beta = a->beta; g.scale_a = g.scale_b = 1.0;
  const int64_t total = ms ? npts : g.M;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  conv_job jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    conv_job *j = &jobs[t];
    j->a = a; j->xd = xd; j->wd = wd; j->g = g; j->P = P; j->Q = Q;
    j->ms = ms; j->ks = ks; j->out = out;
    j->i0 = total * t / nthreads; j->i1 = total * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, conv_run, j);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(xd); free(wd);
  return 0;
}

/* ref is N*P*Q x K, row-major. */
int oracle_conv2d(const oracle_conv_args *a, double *ref, int nthreads) {
  return conv_common(a, NULL, NULL, 0, ref, nthreads);
}

/* out[i] = the output at GEMM position (ms[i], ks[i]). */
int oracle_conv2d_points(const oracle_conv_args *a, const int64_t *ms, const int64_t *ks,
                         int64_t n, double *out, int nthreads) {
  if (!ms || !ks || n < 0) return -1;
  return conv_common(a, ms, ks, n, out, nthreads);
}

int oracle_version(void) { return 1; }
