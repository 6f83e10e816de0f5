// transpose.hip -- layout-driven tiled copy from a row-major M x N source to
// a column-major destination over the same shape, bit for bit:
//     dst[m + n*ld_dst] = src[m*ld_src + n].
//
// Structure from "什么是 CuTe ?" (GPU Glossary zh, 4.21): build the row-major
// source layout and the column-major destination layout over one (M, N)
// shape, tiled_divide both by a block tile, slice out the block's tile, and
// local_partition it among the threads with a thread layout.  The page's
// kernel reads coalesced and writes strided (one element per thread per
// access).  Here both sides move 16 bytes per lane:
//
//   fast path (4-byte elements, M and N multiples of 4, 16-byte aligned rows
//   and columns): the block tile is split into 4x4 micro-tiles; a thread
//   loads its micro-tile as four 16-byte row vectors, transposes it in
//   registers and stores four 16-byte column vectors.  Lanes are laid out
//   8 x 8 over micro-tiles, so every load and every store of a wavefront
//   covers 128-byte runs -- whole cache lines on both sides, no LDS.  All of
//   a thread's loads are issued before any store, to keep many bytes in
//   flight: the copy is bound by HBM bandwidth.
//
//   general path (1/2/4/8/16-byte elements, any pitch, ragged edges): a
//   32 x 32 tile, the page's 8 x 32 row-major thread layout, staged through
//   a padded LDS tile so that reads walk source rows and writes walk
//   destination columns; every access is predicated on the extents.
#include "kernels.hpp"
#include "tla/layout.hpp"

namespace tla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------- fast path
template <int TI, int TJ>
__global__ __launch_bounds__(256) void transpose4_kernel(const uint32_t* __restrict__ src,
                                                        int64_t ld_src, uint32_t* __restrict__ dst,
                                                        int64_t ld_dst, int64_t M, int64_t N,
                                                        int tiles_n) {
  constexpr int TILE_M = 64 * TI, TILE_N = 64 * TJ;
  const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  // global layouts over the same shape, tiled, and this block's tile
  const Layout<2, int64_t> S = row_major<int64_t>(M, N, ld_src);
  const Layout<2, int64_t> DT = col_major<int64_t>(M, N, ld_dst);
  const int64_t blk[2] = {TILE_M, TILE_N};
  const View<2, int64_t> tS = tile_slice(tiled_divide(S, blk), tm, tn);
  const View<2, int64_t> tD = tile_slice(tiled_divide(DT, blk), tm, tn);
  // thread layout over the 16 x 16 micro-tile grid of a 64 x 64 sub-tile:
  // 2 x 2 wavefronts of 8 x 8 lanes, micro-tile row fastest inside a wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mi = (wave & 1) * 8 + (lane & 7);
  const int mj = (wave >> 1) * 8 + (lane >> 3);

  u32x4 v[TI][TJ][4];
#pragma unroll
  for (int a = 0; a < TI; ++a)
#pragma unroll
    for (int b = 0; b < TJ; ++b) {
      const int r = 4 * (mi + 16 * a), c = 4 * (mj + 16 * b);  // micro-tile origin in the tile
      const bool in = tm * TILE_M + r < M && tn * TILE_N + c < N;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (in) v[a][b][q] = __builtin_nontemporal_load((const u32x4*)(src + tS(Coord<2, int64_t>{{r + q, c}})));
    }
#pragma unroll
  for (int a = 0; a < TI; ++a)
#pragma unroll
    for (int b = 0; b < TJ; ++b) {
      const int r = 4 * (mi + 16 * a), c = 4 * (mj + 16 * b);
      if (!(tm * TILE_M + r < M && tn * TILE_N + c < N)) continue;
      const u32x4* x = v[a][b];
      const u32x4 col[4] = {{x[0][0], x[1][0], x[2][0], x[3][0]},
                            {x[0][1], x[1][1], x[2][1], x[3][1]},
                            {x[0][2], x[1][2], x[2][2], x[3][2]},
                            {x[0][3], x[1][3], x[2][3], x[3][3]}};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_nontemporal_store(col[q], (u32x4*)(dst + tD(Coord<2, int64_t>{{r, c + q}})));
    }
}

// -------------------------------------------------------------- general path
template <typename T>
__global__ __launch_bounds__(256) void transpose_tile32_kernel(const T* __restrict__ src,
                                                              int64_t ld_src, T* __restrict__ dst,
                                                              int64_t ld_dst, int64_t M, int64_t N,
                                                              int tiles_n) {
  __shared__ T lds[32][33];
  const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const Layout<2, int64_t> S = row_major<int64_t>(M, N, ld_src);
  const Layout<2, int64_t> DT = col_major<int64_t>(M, N, ld_dst);
  const int64_t blk[2] = {32, 32};
  const View<2, int64_t> tS = tile_slice(tiled_divide(S, blk), tm, tn);
  const View<2, int64_t> tD = tile_slice(tiled_divide(DT, blk), tm, tn);
  const Layout<2, int64_t> thr = row_major<int64_t>(8, 32, 32);  // 8 x 32 threads
  const int64_t tid = threadIdx.x;
  // this thread's elements of the tile: (r + 8i, c), i < 4
  const View<2, int64_t> pS = local_partition(tS, thr, tid);
  const Coord<2, int64_t> tc = compact_inverse(thr, tid);
  const int64_t r = tc.v[0], c = tc.v[1];
  const int64_t mrem = M - tm * 32, nrem = N - tn * 32;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (r + 8 * i < mrem && c < nrem) lds[r + 8 * i][c] = src[pS(Coord<2, int64_t>{{i, 0}})];
  __syncthreads();
  // write side: the same thread layout walks destination columns, so lane c
  // now stands for tile row c and the element is (c, r + 8i)
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (c < mrem && r + 8 * i < nrem) dst[tD(Coord<2, int64_t>{{c, r + 8 * i}})] = lds[c][r + 8 * i];
}

struct alignas(16) B16 {
  uint64_t lo, hi;
};

template <typename T>
int launch_general(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t M, int64_t N,
                   hipStream_t s) {
  const int64_t tm = (M + 31) / 32, tn = (N + 31) / 32;
  if (tm * tn > 0x7FFFFFFF || tn > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(transpose_tile32_kernel<T>, dim3((unsigned)(tm * tn)), dim3(256), 0, s,
                     (const T*)src, ld_src, (T*)dst, ld_dst, M, N, (int)tn);
  return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

int transpose_dispatch(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t M,
                       int64_t N, int eb, hipStream_t s) {
  if (eb == 4 && M % 4 == 0 && N % 4 == 0 && ld_src % 4 == 0 && ld_dst % 4 == 0 && aligned16(src) &&
      aligned16(dst)) {
    // a 64 x 256 block tile: 1 KiB runs per source row and 256-byte runs per
    // destination column in each block; measured fastest of the 4x4-micro-tile
    // shapes on a 16384^2 fp32 copy (taller tiles and multi-tile blocks lose)
    constexpr int TI = 1, TJ = 4;
    const int64_t tm = (M + 64 * TI - 1) / (64 * TI), tn = (N + 64 * TJ - 1) / (64 * TJ);
    if (tm * tn > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((transpose4_kernel<TI, TJ>), dim3((unsigned)(tm * tn)), dim3(256), 0, s,
                       (const uint32_t*)src, ld_src, (uint32_t*)dst, ld_dst, M, N, (int)tn);
    return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
  }
  switch (eb) {
    case 1: return launch_general<uint8_t>(src, ld_src, dst, ld_dst, M, N, s);
    case 2: return launch_general<uint16_t>(src, ld_src, dst, ld_dst, M, N, s);
    case 4: return launch_general<uint32_t>(src, ld_src, dst, ld_dst, M, N, s);
    case 8: return launch_general<uint64_t>(src, ld_src, dst, ld_dst, M, N, s);
    case 16: return launch_general<B16>(src, ld_src, dst, ld_dst, M, N, s);
    default: return TLA_ERR_UNSUPPORTED;
  }
}

}  // namespace tla
