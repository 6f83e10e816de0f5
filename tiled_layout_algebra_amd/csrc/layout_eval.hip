// layout_eval.hip -- runs the device layout module over whole domains so its
// results can be checked one index at a time.
//
//   layout_eval:      out[i] = outer(i)  or  outer(inner(i))
//   thread_map_eval:  the strip-mined thread map the copy kernels use, with
//                     its per-element predicate
//
// Definitions: "Advanced CUTLASS Architecture and Kernel Optimization"
// (oboe.com), "The Algebra of Layouts" (crd2idx as the dot product of
// coordinate and stride) and "Functional Composition" (A o B evaluated as
// A(B(c))); PitchLinearStripminedThreadMap walk-through
// (lpnh.cn/news/2469163), sections 2.1, 3.1-3.4 and 4.2.
#include "kernels.hpp"
#include "tla/copy.hpp"
#include "tla/layout.hpp"

namespace tla {
namespace {

// A runtime flat layout over 64-bit indices: leaf extents and strides.
struct DevLayout {
  int n;
  int64_t shape[TLA_MAX_LEAVES];
  int64_t stride[TLA_MAX_LEAVES];

  // colexicographic idx2crd over the leaves, then the dot product
  __device__ __forceinline__ int64_t operator()(int64_t idx) const {
    int64_t out = 0;
    for (int i = 0; i < n; ++i) {
      const int64_t e = shape[i];
      const int64_t c = idx % e;
      idx /= e;
      out += c * stride[i];
    }
    return out;
  }
};

__global__ __launch_bounds__(256) void layout_eval_kernel(DevLayout outer, DevLayout inner,
                                                         int has_inner, int64_t* __restrict__ out,
                                                         int64_t n) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step)
    out[i] = has_inner ? outer(inner(i)) : outer(i);
}

__global__ __launch_bounds__(256) void thread_map_eval_kernel(StripMinedMap map, int64_t rows_valid,
                                                             int64_t cols_valid,
                                                             int64_t* __restrict__ out_index,
                                                             uint8_t* __restrict__ out_valid) {
  const int total = map.T * map.V * map.I;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    // i = t + T*(v + V*it)
    const int t = i % map.T, v = (i / map.T) % map.V, it = i / (map.T * map.V);
    out_index[i] = map.index(t, it, v);
    if (out_valid) out_valid[i] = map.valid(t, it, v, rows_valid, cols_valid) ? 1 : 0;
  }
}

DevLayout to_dev(const FlatLayout& f) {
  DevLayout d{};
  d.n = f.n;
  for (int i = 0; i < f.n; ++i) {
    d.shape[i] = f.shape[i];
    d.stride[i] = f.stride[i];
  }
  return d;
}

}  // namespace

int layout_eval_dispatch(const FlatLayout& outer, const FlatLayout& inner, bool has_inner,
                         int64_t* out, int64_t n, hipStream_t stream) {
  if (n == 0) return TLA_OK;
  const int64_t blocks = (n + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(layout_eval_kernel, dim3(grid), dim3(256), 0, stream, to_dev(outer),
                     to_dev(inner), has_inner ? 1 : 0, out, n);
  return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
}

int thread_map_eval_dispatch(int R, int C, int T, int V, int I, int contig, int threads_per_row,
                             int swizzle_shift, int64_t rows_valid, int64_t cols_valid,
                             int64_t* out_index, uint8_t* out_valid, hipStream_t stream) {
  const StripMinedMap map(R, C, T, V, I, contig, threads_per_row, swizzle_shift);
  const int64_t total = (int64_t)T * V * I;
  if (total == 0) return TLA_OK;
  const int64_t blocks = (total + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(thread_map_eval_kernel, dim3(grid), dim3(256), 0, stream, map, rows_valid,
                     cols_valid, out_index, out_valid);
  return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
}

}  // namespace tla
