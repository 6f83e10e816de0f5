// transpose.hip -- layout-driven tiled copy from a row-major M x N source to
// a column-major destination over the same shape, bit for bit:
//     dst[m + n*ld_dst] = src[m*ld_src + n].
//
// Both tensors are described as layouts over one (M, N) shape ("什么是 CuTe
// ?", GPU Glossary zh, 4.21): the source row-major with pitch ld_src, the
// destination column-major with pitch ld_dst.  tiled_divide by the block
// tile and a slice at the block's tile index give each block its tile of
// both tensors; the element offsets inside the tile come from the same
// layouts.  The page's kernel reads coalesced and writes strided (one
// element per thread per access); here both sides move whole cache lines:
//
//   fast path (4-byte elements, M and N multiples of 4, 16-byte aligned rows
//   and columns): the 64 x 256 block tile is cut into 4x4 micro-tiles; a
//   thread loads its micro-tile as four 16-byte row vectors, transposes it
//   in registers and stores four 16-byte column vectors.  Lanes are laid out
//   8 x 8 over micro-tiles, so every wavefront load and store covers
//   128-byte runs -- whole cache lines on both sides, no LDS.  All of a
//   thread's loads are issued before any store; whole tiles carry no
//   predicate at all (one exec-mask branch per access measured 416.8 us
//   against 394 us on a 16384^2 fp32 transpose), edge tiles check each
//   micro-tile.
//
//   general path (1/2/4/8/16-byte elements, any pitch, ragged edges): a
//   32 x 32 tile staged through a padded LDS tile.  The strip-mined thread
//   map of the PitchLinearStripminedThreadMap walk-through (sections 2.1,
//   3.4) places the 256 threads: its row-contiguous form for the reads
//   (consecutive threads along a source row) and its column-contiguous form
//   for the writes (consecutive threads down a destination column); every
//   element access is predicated on the extents.
#include "kernels.hpp"
#include "tla/copy.hpp"
#include "tla/layout.hpp"

namespace tla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------- fast path
// One thread's TI x TJ micro-tiles: rows 4*(mi + 16a), columns 4*(mj + 16b)
// of the block tile, lanes 8 x 8 per wave, waves 2 x 2.
template <int TI, int TJ, bool kEdge>
__device__ __forceinline__ void transpose_micro(const uint32_t* __restrict__ s, int64_t ld_src,
                                                uint32_t* __restrict__ d, int64_t ld_dst,
                                                int64_t rows_left, int64_t cols_left, int mi,
                                                int mj) {
  u32x4 v[TI][TJ][4];
#pragma unroll
  for (int a = 0; a < TI; ++a)
#pragma unroll
    for (int b = 0; b < TJ; ++b) {
      const int r = 4 * (mi + 16 * a), c = 4 * (mj + 16 * b);
      if (kEdge && !(r < rows_left && c < cols_left)) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[a][b][q] = __builtin_nontemporal_load((const u32x4*)(s + (r + q) * ld_src + c));
    }
#pragma unroll
  for (int a = 0; a < TI; ++a)
#pragma unroll
    for (int b = 0; b < TJ; ++b) {
      const int r = 4 * (mi + 16 * a), c = 4 * (mj + 16 * b);
      if (kEdge && !(r < rows_left && c < cols_left)) continue;
      const u32x4* x = v[a][b];
      const u32x4 col[4] = {{x[0][0], x[1][0], x[2][0], x[3][0]},
                            {x[0][1], x[1][1], x[2][1], x[3][1]},
                            {x[0][2], x[1][2], x[2][2], x[3][2]},
                            {x[0][3], x[1][3], x[2][3], x[3][3]}};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_nontemporal_store(col[q], (u32x4*)(d + (c + q) * ld_dst + r));
    }
}

template <int TI, int TJ>
__global__ __launch_bounds__(256) void transpose4_kernel(const uint32_t* __restrict__ src,
                                                        int64_t ld_src, uint32_t* __restrict__ dst,
                                                        int64_t ld_dst, int64_t M, int64_t N,
                                                        int tiles_n) {
  constexpr int TILE_M = 64 * TI, TILE_N = 64 * TJ;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  // this block's tile of both layouts: the tile origins are scalars, the
  // inside-tile strides are (ld_src, 1) and (1, ld_dst)
  const int64_t blk[2] = {TILE_M, TILE_N};
  const View<2, int64_t> tS = tile_slice(tiled_divide(row_major<int64_t>(M, N, ld_src), blk), (int64_t)tm, (int64_t)tn);
  const View<2, int64_t> tD = tile_slice(tiled_divide(col_major<int64_t>(M, N, ld_dst), blk), (int64_t)tm, (int64_t)tn);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mi = (wave & 1) * 8 + (lane & 7);
  const int mj = (wave >> 1) * 8 + (lane >> 3);
  const int64_t rows_left = M - (int64_t)tm * TILE_M, cols_left = N - (int64_t)tn * TILE_N;
  if (rows_left >= TILE_M && cols_left >= TILE_N)
    transpose_micro<TI, TJ, false>(src + tS.offset, tS.layout.stride[0], dst + tD.offset,
                                   tD.layout.stride[1], rows_left, cols_left, mi, mj);
  else
    transpose_micro<TI, TJ, true>(src + tS.offset, tS.layout.stride[0], dst + tD.offset,
                                  tD.layout.stride[1], rows_left, cols_left, mi, mj);
}

// -------------------------------------------------------------- general path
template <typename T>
__global__ __launch_bounds__(256) void transpose_tile32_kernel(const T* __restrict__ src,
                                                              int64_t ld_src, T* __restrict__ dst,
                                                              int64_t ld_dst, int64_t M, int64_t N,
                                                              int tiles_n) {
  __shared__ T lds[32][33];
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int64_t blk[2] = {32, 32};
  const View<2, int64_t> tS = tile_slice(tiled_divide(row_major<int64_t>(M, N, ld_src), blk), (int64_t)tm, (int64_t)tn);
  const View<2, int64_t> tD = tile_slice(tiled_divide(col_major<int64_t>(M, N, ld_dst), blk), (int64_t)tm, (int64_t)tn);
  const int64_t rows_left = M - (int64_t)tm * 32, cols_left = N - (int64_t)tn * 32;
  // 32 x 32 tile, 256 threads, one element per access, four accesses each
  constexpr StripMinedMap rd(32, 32, 256, 1, 4, 1);   // threads along a row
  constexpr StripMinedMap wr(32, 32, 256, 1, 4, 0);   // threads down a column
  static_assert(rd.well_formed() && wr.well_formed(), "tile thread maps");
  const int t = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = rd.row(t, it, 0), c = rd.col(t, it, 0);
    if (r < rows_left && c < cols_left) lds[r][c] = src[tS(Coord<2, int64_t>{{r, c}})];
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = wr.row(t, it, 0), c = wr.col(t, it, 0);
    if (r < rows_left && c < cols_left) dst[tD(Coord<2, int64_t>{{r, c}})] = lds[r][c];
  }
}

// ------------------------------------------------------------- 2-D copy
// Row-major to row-major: block b copies a chunk of 256 vectors (or
// elements) of row b / chunks, one per thread -- on a 16384^2 fp32 copy one
// 16-byte vector per thread measured 6.55 TB/s, against 5.9-6.2 with 2 to 8
// vectors per thread and 5.2 with 16.
template <typename V>
__global__ __launch_bounds__(256) void copy_rows_kernel(const V* __restrict__ src, int64_t ld_src,
                                                       V* __restrict__ dst, int64_t ld_dst,
                                                       int64_t row_len, int64_t chunks) {
  const int64_t row = blockIdx.x / chunks, chunk = blockIdx.x - row * chunks;
  const int64_t i = chunk * 256 + threadIdx.x;
  if (i < row_len)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + row * ld_src + i),
                                dst + row * ld_dst + i);
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

template <typename V>
int launch_copy(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t M,
                int64_t row_len, hipStream_t s) {
  const int64_t chunks = (row_len + 255) / 256;
  if (M * chunks > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(copy_rows_kernel<V>, dim3((unsigned)(M * chunks)), dim3(256), 0, s,
                     (const V*)src, ld_src, (V*)dst, ld_dst, row_len, chunks);
  return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
}

}  // namespace

int transpose_dispatch(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t M,
                       int64_t N, int eb, hipStream_t s) {
  if (eb == 4 && M % 4 == 0 && N % 4 == 0 && ld_src % 4 == 0 && ld_dst % 4 == 0 && aligned16(src) &&
      aligned16(dst)) {
    // a 64 x 256 block tile: 1 KiB runs per source row and 256-byte runs per
    // destination column in each block.  On a 16384^2 fp32 transpose it was
    // the fastest shape of the 4x4-micro-tile family (GB/s): 64x256 5455,
    // 128x256 5230, 64x512 5254, 128x128 4801, 64x128 5023, 256x64 4306,
    // 64x64 4211; walking tile rows fastest in launch order or laying lanes
    // 16 x 4 lost 10-20 %.  A plain streaming copy of the same bytes runs at
    // 6516-6553 GB/s on the same box.
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

int copy_dispatch(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t M,
                  int64_t N, int eb, hipStream_t s) {
  // whole 16-byte vectors when every row starts 16-byte aligned
  const int64_t row_bytes = N * eb;
  if (row_bytes % 16 == 0 && (ld_src * eb) % 16 == 0 && (ld_dst * eb) % 16 == 0 &&
      aligned16(src) && aligned16(dst))
    return launch_copy<u32x4>(src, ld_src * eb / 16, dst, ld_dst * eb / 16, M, row_bytes / 16, s);
  switch (eb) {
    case 1: return launch_copy<uint8_t>(src, ld_src, dst, ld_dst, M, N, s);
    case 2: return launch_copy<uint16_t>(src, ld_src, dst, ld_dst, M, N, s);
    case 4: return launch_copy<uint32_t>(src, ld_src, dst, ld_dst, M, N, s);
    case 8: return launch_copy<uint64_t>(src, ld_src, dst, ld_dst, M, N, s);
    case 16: return launch_copy<u32x4>(src, ld_src, dst, ld_dst, M, N, s);
    default: return TLA_ERR_UNSUPPORTED;
  }
}

}  // namespace tla
