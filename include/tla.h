/*
 * tla.h -- C ABI of libtla.so: a layout-algebra-driven tiled GEMM with a
 * fused epilogue, a layout-driven tiled transpose, and a device evaluator
 * of shape/stride layouts, for AMD Instinct MI355X (gfx950 / CDNA4).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Plain C types only.  Device pointers are raw HIP device addresses;
 *   `stream` is a hipStream_t passed as void* (NULL = the null stream).
 * - Ownership: the caller owns every buffer.  The library never allocates,
 *   frees or retains user memory, keeps no global state and needs no
 *   workspace, so it is reentrant.
 * - Asynchrony: device work is enqueued on `stream` and the call returns.
 *   Argument errors are reported synchronously (no work is enqueued);
 *   execution faults surface at the caller's next synchronisation.
 * - Status codes: TLA_OK (0) or a negative TLA_ERR_* value; no exceptions
 *   cross the boundary.  tla_status_string() names them.
 * - Sizes, leading dimensions and strides are counted in ELEMENTS.
 *
 * Sources of the operations (page titles and sections):
 * - "CUTLASS / CuTe 主线" (hpc.payai.win/cutlass): section 一 maps
 *   C[M,N] = A[M,K] x B[K,N] onto block / warp / instruction tiles and
 *   ends in an epilogue (alpha/beta, bias/activation, store); section 二
 *   describes the host entry as close to cuBLAS; section 三's Collective
 *   Epilogue fuses scale/bias/activation; lesson 7 of its course table is
 *   mixed precision with an fp32 accumulator.
 * - "什么是 CuTe ?" (GPU Glossary zh, 4.21): the transpose of a row-major
 *   tensor into a column-major one over the same shape, by tiles.
 * - "Advanced CUTLASS Architecture and Kernel Optimization" (oboe.com),
 *   "The Algebra of Layouts", "Functional Composition", "Advanced Layout
 *   Operations": Layout = (Shape, Stride), crd2idx, composition,
 *   logical_divide.
 * - PitchLinearStripminedThreadMap walk-through (lpnh.cn/news/2469163),
 *   sections 2.1, 3.1-3.4, 4.2: the strip-mined thread map, its tile
 *   equation and its predicate; section 6.3: the pitch comes from the
 *   tensor layout.
 */
#ifndef TLA_H
#define TLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------- status */
enum {
  TLA_OK = 0,
  TLA_ERR_INVALID_ARG = -1, /* NULL pointer, negative size, ld too small,
                               C == NULL with beta != 0, n != domain size,
                               tile equation violated, ...            */
  TLA_ERR_UNSUPPORTED = -2, /* dtype / order combination not provided */
  TLA_ERR_OVERLAP = -3,     /* transpose source and destination overlap */
  TLA_ERR_HIP = -4          /* kernel launch failed (hipGetLastError is
                               consumed by the call)                   */
};

/* ------------------------------------------------------- element types */
typedef enum {
  TLA_F16 = 0,  /* IEEE binary16                                        */
  TLA_BF16 = 1, /* bfloat16                                             */
  TLA_E4M3 = 2, /* OCP FP8 E4M3FN (bias 7, max 448, no inf)             */
  TLA_F32 = 3   /* IEEE binary32 (bias / C only)                        */
} tla_dtype;

typedef enum { TLA_ROW_MAJOR = 0, TLA_COL_MAJOR = 1 } tla_order;

typedef enum {
  TLA_ACT_NONE = 0,
  TLA_ACT_RELU = 1, /* max(y, 0)                                        */
  TLA_ACT_GELU = 2  /* y * Phi(y), the erf form                         */
} tla_act;

/* -------------------------------------------------------------- GEMM */
/*
 * D = act( alpha*scale_a*scale_b * (A . B)  +  beta*C  +  bias )
 *
 * Logical shapes: A is M x K, B is K x N, C and D are M x N; bias has N
 * entries (one per output column) or is NULL.  Each matrix has its own
 * storage order and leading dimension: element (r, c) of a row-major
 * matrix is at r*ld + c, of a column-major one at r + c*ld; ld must be at
 * least the contiguous extent (and >= 1).
 *
 * Arithmetic: products of the A/B storage values are accumulated in fp32;
 * the epilogue runs in fp32 (alpha_eff = alpha*scale_a*scale_b, then
 * + beta*C(m,n) when beta != 0, + bias[n] when bias != NULL, then act) and
 * rounds to D's type to nearest even.  C is not read when beta == 0 (it may
 * then be NULL).  scale_a / scale_b are the per-tensor dequantisation
 * scales of fp8 operands (pass 1 otherwise).
 *
 * Supported combinations:
 *   A, B:  both F16, both BF16, or both E4M3
 *   D:     F16 or BF16;  C and bias: F16, BF16 or F32
 *   any order for A, B, C, D; any leading dimension; any alignment
 *   (aligned, K-contiguous operands take the fast path, the rest a general
 *   predicated path with the same results up to fp32 summation order).
 *
 * Edge cases: M == 0 or N == 0 is a no-op returning TLA_OK; K == 0 gives
 * D = act(beta*C + bias).  D may alias C only with identical order and
 * leading dimension.  Elements of D's padding (ld beyond the extent) are
 * never written; elements of A, B, C padding are never read.
 */
typedef struct {
  int64_t M, N, K;
  const void *A; int32_t a_type; int32_t a_order; int64_t lda;
  const void *B; int32_t b_type; int32_t b_order; int64_t ldb;
  const void *C; int32_t c_type; int32_t c_order; int64_t ldc;
  void *D;       int32_t d_type; int32_t d_order; int64_t ldd;
  const void *bias; int32_t bias_type;
  int32_t act;   /* tla_act */
  float alpha, beta, scale_a, scale_b;
} tla_gemm_args;

int tla_gemm_epilogue(const tla_gemm_args *args, void *stream);

/* Name of the kernel variant tla_gemm_epilogue would launch for `args`
 * (written NUL-terminated into buf, at most cap bytes).  Host only. */
int tla_gemm_variant(const tla_gemm_args *args, char *buf, int32_t cap);

/*
 * Tile-configuration dispatch ("CUTLASS / CuTe 主线", the kernel-composition
 * and profiling lesson; the ThreadblockShape trade-off between reuse and
 * occupancy).  The library compiles TLA_GEMM_VARIANTS kernels:
 *   0 "gemm_pingpong_256x256" 256x256 tiles, 8 wavefronts in two groups of
 *                            four (2x2 waves of 64x128 each) that take turns
 *                            between MFMA-only and memory phases; direct
 *                            global->LDS copies; every operand type (16-bit
 *                            operands may also have an N-contiguous B or an
 *                            M-contiguous A, as for variant 1)
 *   1 "gemm_fast_128x128"    128x128 tiles, direct copies (16-bit: 8
 *                            wavefronts of 64x32; e4m3: 4 of 64x64); for
 *                            16-bit operands B may also be N-contiguous
 *                            (row-major K x N) and A M-contiguous
 *                            (column-major M x K): their fragments are then
 *                            read through LDS transpose reads
 *   2 "gemm_general_128x128" 128x128 tiles, 4 wavefronts, register-staged
 *                            predicated loads: any order, pitch, alignment,
 *                            ragged K
 *   3 "gemm_fast_256x256"    256x256 tiles, one group (16-bit: 8 wavefronts
 *                            of 128x64; e4m3: 4 of 128x128), direct copies
 * tla_gemm_epilogue picks one from the problem: in the fast layout, the
 * N-contiguous-B and the M-contiguous-A layouts, variant 0 with at least
 * 128 tiles of 256x256 and 1 otherwise; variant 2 outside them;
 * tla_gemm_run_variant runs the one asked for, with the same semantics and
 * tolerance, or returns TLA_ERR_UNSUPPORTED when a fast variant is asked
 * for a problem without the fast layout (both operands K-contiguous,
 * 16-byte aligned rows, K a multiple of 8 for 16-bit operands or of 16 for
 * e4m3 -- the last k-tile may end inside the slab -- each operand < 2 GiB;
 * e4m3 variants 1 and 3 need K a multiple of 128, and the automatic choice
 * for e4m3 below 128 tiles with other K is variant 2) -- variants 0 and 1
 * also accept the N-contiguous-B layout (16-bit operands; A as in the fast
 * layout; B row-major with 16-byte aligned rows, N and K multiples of 8, B
 * below 2 GiB) and the M-contiguous-A layout (16-bit operands; A
 * column-major with 16-byte aligned columns, M and K multiples of 8, A
 * below 2 GiB; B in either of the layouts above).
 * Variant ids outside [0, TLA_GEMM_VARIANTS) are TLA_ERR_INVALID_ARG.
 */
#define TLA_GEMM_VARIANTS 4
int tla_gemm_run_variant(const tla_gemm_args *args, int32_t variant, void *stream);

/* A variant's compiled kernel for operand type a_type, as the HIP runtime
 * reports it on the current device: threads per workgroup, static LDS bytes,
 * vector registers per lane and the number of workgroups that can be
 * resident on one compute unit.  Needs a device (TLA_ERR_HIP without). */
typedef struct {
  char name[32];
  int32_t block_m, block_n, threads;
  int32_t lds_bytes, vgprs, blocks_per_cu;
} tla_gemm_kernel_info;
int tla_gemm_variant_info(int32_t variant, int32_t a_type, tla_gemm_kernel_info *out);

/* --------------------------------------------------------- transpose */
/*
 * dst(m, n) = src(m, n) bit for bit, from a row-major source to a
 * column-major destination over the same M x N shape:
 *     dst[m + n*ld_dst] = src[m*ld_src + n]      (element units)
 * elem_bytes: 1, 2, 4, 8 or 16; ld_src >= N, ld_dst >= M.  Elements are
 * moved as raw bits (NaN payloads and subnormals are preserved).  The
 * source and destination byte ranges must not overlap (TLA_ERR_OVERLAP).
 * M == 0 or N == 0 is a no-op.  Destination padding is never written.
 */
int tla_tiled_transpose(const void *src, int64_t ld_src, void *dst, int64_t ld_dst,
                        int64_t M, int64_t N, int32_t elem_bytes, void *stream);

/*
 * The identity-layout case of the same layout-driven copy: a row-major
 * M x N source to a row-major destination, bit for bit,
 *     dst[m*ld_dst + n] = src[m*ld_src + n]      (element units)
 * ("什么是 CuTe ?": a copy between two layouts over one shape; here both
 * are row-major).  It moves the same bytes as tla_tiled_transpose with
 * unit-stride runs on both sides, so it gives the memory-system ceiling a
 * transpose is measured against.  elem_bytes: 1, 2, 4, 8 or 16; ld_src >= N,
 * ld_dst >= N; element-aligned pointers (TLA_ERR_INVALID_ARG otherwise);
 * non-overlapping byte ranges (TLA_ERR_OVERLAP).  M == 0 or N == 0 is a
 * no-op; destination padding is never written.
 */
int tla_tiled_copy(const void *src, int64_t ld_src, void *dst, int64_t ld_dst,
                   int64_t M, int64_t N, int32_t elem_bytes, void *stream);

/* ------------------------------------------------------ convolution */
/*
 * Forward convolution as an implicit GEMM (PitchLinearStripminedThreadMap
 * walk-through, section 5.2: one GEMM dimension is the output pixel, the
 * other the filter position times the channel).  Cross-correlation:
 *   y[n,p,q,k] = act(alpha * sum_{r,s,c} x[n, p*u - ph + r*dh, q*v - pw + s*dw, c]
 *                                     * w[k, r, s, c]
 *                    + beta * C[n,p,q,k] + bias[k])
 * with x taken as 0 outside the image, accumulated in fp32 and rounded to
 * nearest even.  x is N x H x W x C (NHWC), w is K x R x S x C (KRSC), y and
 * C are N x P x Q x K (NPQK), all dense and of one type (f16 or bf16); bias
 * (length K, f16/bf16/f32) may be NULL; C may be NULL when beta == 0 and may
 * alias y.  P = (H + 2 ph - dh (R-1) - 1) / u + 1 and Q likewise (floor).
 * The GEMM has M = N*P*Q, N = K, K = R*S*C; each of them must stay below
 * 2^31, and so must N*H*W*C; the padded extents H + 2 ph and W + 2 pw must
 * stay below 2^30.  N == 0, P < 1 or Q < 1 is a no-op.  Strides and dilations must be
 * >= 1, paddings >= 0, extents >= 1 (TLA_ERR_INVALID_ARG otherwise).
 */
typedef struct {
  int64_t N, H, W, C, K, R, S;
  int32_t stride_h, stride_w, pad_h, pad_w, dil_h, dil_w;
  const void *x;
  const void *w;
  const void *C_res;
  void *y;
  int32_t type;
  const void *bias;
  int32_t bias_type;
  int32_t act;
  float alpha, beta;
} tla_conv2d_args;

int tla_conv2d_fprop(const tla_conv2d_args *args, void *stream);

/* The convolution kernels, for comparison and testing:
 *   0 "conv_slab"            64 input and 64 output channels at stride 1:
 *                            the whole filter and the image rows of a band
 *                            of output rows in LDS, each copied in once
 *                            (x and w 16-byte aligned, H*W*128 < 2^31, a
 *                            band of whole output rows fitting LDS)
 *   1 "conv_implicit_fast"   the implicit GEMM with direct-to-LDS copies (C
 *                            a multiple of 64, x and w 16-byte aligned, x
 *                            and w each below 2 GiB)
 *   2 "conv_implicit_general" the implicit GEMM with register-staged,
 *                            predicated loads: any shape
 * tla_conv2d_fprop picks the first one that applies;
 * tla_conv2d_fprop_variant runs the one asked for, with the same semantics
 * and tolerance, or returns TLA_ERR_UNSUPPORTED when the problem does not
 * meet its conditions.  Arguments are validated as for tla_conv2d_fprop;
 * variant ids outside [0, TLA_CONV_VARIANTS) are TLA_ERR_INVALID_ARG.
 */
#define TLA_CONV_VARIANTS 3
int tla_conv2d_fprop_variant(const tla_conv2d_args *args, int32_t variant, void *stream);

/* ---------------------------------------------------------- layouts */
/*
 * A shape/stride layout with at most one level of nesting: n_modes
 * top-level modes, mode i made of leaves[i] leaves (1 = a plain integer
 * mode); shape[] and stride[] list the leaf extents and strides mode by
 * mode.  A 1-D index walks the layout colexicographically (first leaf
 * fastest), and the value is the dot product of the leaf coordinates with
 * the strides.  Extents must be >= 1.
 *
 * Example: the SM80 A-operand TV layout ((4,8),(2,2,2)):((32,1),(16,8,128))
 * is n_modes 2, leaves {2,3}, shape {4,8,2,2,2}, stride {32,1,16,8,128}.
 */
#define TLA_MAX_MODES 8
#define TLA_MAX_LEAVES 16
typedef struct {
  int32_t n_modes;
  int32_t leaves[TLA_MAX_MODES];
  int64_t shape[TLA_MAX_LEAVES];
  int64_t stride[TLA_MAX_LEAVES];
} tla_layout;

/* Number of coordinates (product of all leaf extents).  Host only. */
int tla_layout_size(const tla_layout *L, int64_t *size);

/*
 * out[i] = outer(i)             for i < n, when inner == NULL (n == size(outer))
 * out[i] = outer(inner(i))      for i < n, otherwise       (n == size(inner))
 * Composition is pointwise: inner's value is a 1-D index into outer's
 * domain, so every inner(i) must lie in [0, size(outer)) -- checked on the
 * host from the range of inner.  `out` is a device array of n int64.
 */
int tla_layout_eval(const tla_layout *outer, const tla_layout *inner, int64_t *out,
                    int64_t n, void *stream);

/*
 * logical_divide of a flat layout (every mode one leaf) by a tile shape:
 * mode i of extent n_i and stride d_i becomes the nested mode
 * (tile_i, ceil(n_i/tile_i)) : (d_i, d_i*tile_i) -- position inside the
 * tile first, tile index second.  n_tile == n_modes.  Host only.
 */
int tla_logical_divide(const tla_layout *L, const int64_t *tile, int32_t n_tile,
                       tla_layout *out);

/*
 * tiled_divide: logical_divide, then the inside-tile leaves gathered into
 * mode 0 and each tile-index leaf a mode of its own:
 * ((tile_0, tile_1, ...), rest_0, rest_1, ...).  Host only.
 */
int tla_tiled_divide(const tla_layout *L, const int64_t *tile, int32_t n_tile,
                     tla_layout *out);

/*
 * The strip-mined thread map of an R x C tile, T threads, V contiguous
 * elements per access, I iterations per thread, as a TV layout
 *   ((G, T/G), (V, I)) : ((V, Q), (1, S*Q))
 * into the tile index, with Q the contiguous extent (C when
 * contiguous_dim == 1: index row*C + col; R when contiguous_dim == 0:
 * index row + col*R), G = Q/V column groups, S = (strided extent)/I the
 * row stride.  Requires R*C == T*V*I, V | Q, G | T and S == T/G
 * (TLA_ERR_INVALID_ARG otherwise).  Host only.
 */
int tla_thread_map(int64_t R, int64_t C, int32_t T, int32_t V, int32_t I,
                   int32_t contiguous_dim, tla_layout *out);

/*
 * Runs the device-side strip-mined thread map the copy kernels use, for
 * every (t, it, v) with t < T, it < I, v < V, at index
 * i = t + T*(v + V*it):
 *   out_index[i] = tile index of the element (as tla_thread_map),
 *   out_valid[i] = 1 if the element lies inside the first rows_valid rows
 *                  and cols_valid columns of the tile, else 0.
 * out_index: device int64[T*V*I]; out_valid: device uint8[T*V*I] or NULL.
 * Same argument rules as tla_thread_map; rows_valid, cols_valid >= 0.
 */
int tla_thread_map_eval(int64_t R, int64_t C, int32_t T, int32_t V, int32_t I,
                        int32_t contiguous_dim, int64_t rows_valid, int64_t cols_valid,
                        int64_t *out_index, uint8_t *out_valid, void *stream);

/*
 * The two optional parameters of the same walk-through (0 / -1 = off; the
 * plain functions above are these with both off):
 *  - threads_per_row G (section 2.2, which lets a parameter override the
 *    default thread distribution): G threads share one strided position
 *    instead of Q/V; a thread then makes Ic = (Q/V)/G passes along the
 *    contiguous dimension (innermost) per strided step:
 *      column group = (t mod G) + G*(it mod Ic),
 *      strided      = t div G + (it div Ic)*S,   S = T/G,
 *    requiring G | Q/V, G | T, Ic | I and P == S*(I/Ic);
 *  - swizzle_shift s >= 0 (section 5.3, a map that exchanges bits of the
 *    thread-to-address mapping to spread bank conflicts): the column group
 *    is XORed with (strided >> s) mod (Q/V), Q/V a power of two -- a
 *    permutation of the groups at every strided position.
 * tla_thread_map_ex returns the unswizzled map's TV layout
 *   ((G, T/G), (V, Ic, I/Ic)) : ((V, Q), (1, G*V, S*Q))
 * (the two-leaf value mode of tla_thread_map when Ic == 1); a swizzled map
 * is not a shape/stride layout and is only evaluated on the device.
 * TLA_ERR_INVALID_ARG when a requirement fails.
 */
int tla_thread_map_ex(int64_t R, int64_t C, int32_t T, int32_t V, int32_t I,
                      int32_t contiguous_dim, int32_t threads_per_row, tla_layout *out);
int tla_thread_map_eval_ex(int64_t R, int64_t C, int32_t T, int32_t V, int32_t I,
                           int32_t contiguous_dim, int32_t threads_per_row, int32_t swizzle_shift,
                           int64_t rows_valid, int64_t cols_valid, int64_t *out_index,
                           uint8_t *out_valid, void *stream);

/* ------------------------------------------------ layout algebra (host) */
/*
 * logical_product of two layouts, in the reading "Advanced CUTLASS
 * Architecture and Kernel Optimization", "Advanced Layout Operations" gives
 * it: the result's shape and stride are the concatenations of the inputs'.
 * out has L's modes followed by M's (n_modes(L) + n_modes(M) <= 8, leaves
 * <= 16), so as a function of the 1-D index
 *   out(i) = L(i mod size(L)) + M(i / size(L)).
 * TLA_ERR_INVALID_ARG for a malformed input or a result past the limits.
 */
int tla_logical_product(const tla_layout *L, const tla_layout *M, tla_layout *out);

/*
 * The flattest layout with L's function: every leaf of extent 1 dropped and
 * neighbouring leaves merged while stride[k+1] == shape[k] * stride[k].
 * out is flat (one leaf per mode) when at most 8 leaves remain, else one
 * mode holding them all; out(i) == L(i) for every i < size(L), and no two
 * neighbouring leaves of out could merge again.  A layout of size 1 becomes
 * 1:0.  Host only.
 */
int tla_coalesce(const tla_layout *L, tla_layout *out);

/*
 * A o B in closed form ("Functional Composition": c -> A(B(c))): a layout R
 * with B's top-level modes such that R(i) == A(B(i)) for every i < size(B),
 * A taking B's value as a 1-D index.  Every B(i) must lie in
 * [0, size(A)) (TLA_ERR_INVALID_ARG otherwise, as for tla_layout_eval).
 * Each leaf s:d of B becomes the run of A's (coalesced) modes that the
 * indices 0, d, ..., (s-1)d walk: d must be a product of whole leading
 * extents of A times a divisor of the next one, and s must end on or
 * inside a mode boundary the same way; the leaves of B must cover disjoint
 * ranges of A's mixed radix (sorted by stride, d' >= d*s), so that A adds
 * their contributions without carries.  When these hold the closed form is
 * exact; otherwise TLA_ERR_UNSUPPORTED (use the pointwise tla_layout_eval).
 * TLA_ERR_UNSUPPORTED also when the result needs more than 16 leaves.
 */
int tla_composition(const tla_layout *A, const tla_layout *B, tla_layout *out);

/*
 * logical_divide of every mode, nested modes included: mode i of L (size
 * n_i, any nesting) and tile t_i give two top-level modes of out, the
 * position inside the tile and the tile index, in the order
 * (inside_0, index_0, inside_1, index_1, ...) -- 2 * n_modes(L) <= 8.
 * inside_i (e < t_i) and index_i (q < ceil(n_i / t_i)) stand for the
 * element at 1-D position e + t_i * q of mode i.  A nested mode is divided
 * by composing it with (t_i, n_i/t_i):(1, t_i), so t_i must divide n_i and
 * the composition must have a closed form (TLA_ERR_UNSUPPORTED otherwise);
 * a one-leaf mode n:d may be divided raggedly into (t_i:d,
 * ceil(n/t_i):d*t_i), the last tile reaching past the end.  Host only.
 */
int tla_logical_divide_modes(const tla_layout *L, const int64_t *tile, int32_t n_tile,
                             tla_layout *out);

/* ------------------------------------------------------------- misc */
const char *tla_status_string(int status);
int tla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TLA_H */
