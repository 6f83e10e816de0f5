// kernels.hpp -- internal launch interface between the C ABI (api.cpp) and
// the HIP kernel files.  Every function here assumes its arguments were
// validated by the ABI layer and returns a TLA_* status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tla.h"

namespace tla {

// A validated GEMM problem, in the element units of each operand.
struct GemmProblem {
  int64_t M, N, K;
  const void* A; int a_type; int a_order; int64_t lda;
  const void* B; int b_type; int b_order; int64_t ldb;
  const void* C; int c_type; int c_order; int64_t ldc;
  void* D; int d_type; int d_order; int64_t ldd;
  const void* bias; int bias_type;
  int act;
  float alpha_eff;  // alpha * scale_a * scale_b
  float beta;
};

// Picks the kernel variant; launches it unless `dry_run`.  `name` receives
// the variant's name (may be NULL).
// Forward convolution as an implicit GEMM: x N x H x W x C_in (NHWC), w K x
// R x S x C_in (KRSC), y and C N x P x Q x K (NPQK); all of one 16-bit type.
struct ConvProblem {
  int64_t N, H, W, C_in, K, R, S, P, Q;
  int u, v, ph, pw, dh, dw;
  const void* x; const void* w; const void* C; void* y;
  int type;
  const void* bias; int bias_type;
  int act;
  float alpha, beta;
};
// forced = -1 picks the kernel (slab, implicit direct-to-LDS, implicit
// register-staged: the first that applies); 0..2 runs that one or returns
// TLA_ERR_UNSUPPORTED.
int conv_dispatch(const ConvProblem& c, hipStream_t stream, int forced = -1);

// GEMM kernel variants: 0 two-group 256x256, 1 fast 128x128, 2 general
// 128x128, 3 single-group 256x256.
constexpr int kGemmVariants = 4;
struct GemmKernelInfo {
  const char* name;
  int tile, threads, lds_bytes, vgprs, blocks_per_cu;
};
// forced = -1 picks the variant from the problem; a forced fast variant on a
// problem without the fast layout returns TLA_ERR_UNSUPPORTED.
int gemm_dispatch(const GemmProblem& p, hipStream_t stream, bool dry_run, const char** name,
                  int forced = -1);
int gemm_variant_info(int a_type, int variant, GemmKernelInfo* out);

int transpose_dispatch(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t M,
                       int64_t N, int elem_bytes, hipStream_t stream);
int copy_dispatch(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t M,
                  int64_t N, int elem_bytes, hipStream_t stream);

// Flat leaf lists of (validated) layouts; inner_leaves == 0 means no inner.
struct FlatLayout {
  int n;
  int64_t shape[TLA_MAX_LEAVES];
  int64_t stride[TLA_MAX_LEAVES];
};
int layout_eval_dispatch(const FlatLayout& outer, const FlatLayout& inner, bool has_inner,
                         int64_t* out, int64_t n, hipStream_t stream);

int thread_map_eval_dispatch(int R, int C, int T, int V, int I, int contig, int threads_per_row,
                             int swizzle_shift, int64_t rows_valid, int64_t cols_valid,
                             int64_t* out_index, uint8_t* out_valid, hipStream_t stream);

}  // namespace tla
