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
//   and columns): 256 x 64 block tiles, staged through LDS.  A thread loads
//   4x4 micro-tiles as four 16-byte row vectors, 16 lanes side by side along
//   each source row (256-byte runs), transposes each micro-tile in registers
//   and writes its four 16-byte column pieces into LDS, which holds the tile
//   column by column; then 64 lanes read one whole LDS column each and store
//   it as a 1 KiB run of a destination column.  Tiles are launched tile row
//   fastest, so consecutive workgroups continue the same destination
//   columns.  All of a thread's loads are issued before any store; whole
//   tiles carry no predicate, edge tiles check each micro-tile and chunk.
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
// Block tile TM x TN of 4-byte elements, 256 threads.  Load: thread t owns
// micro-tile column mj = t % NT and micro-tile rows t / NT + k * (256 / NT).
// LDS: TN rows (one per tile column) of MT 16-byte chunks (chunk i = tile
// rows 4i..4i+3), chunk i of row c stored at position i ^ ((c / 4) % MT): the
// 16 lanes of one write phase then hit 16 distinct bank groups, and a row
// stays a permutation of its chunks for the conflict-free read.  Store:
// thread t moves chunk t % MT of LDS rows t / MT + k * (256 / MT).
template <int TM, int TN, bool kEdge>
__device__ __forceinline__ void transpose_tile(const uint32_t* __restrict__ s, int64_t ld_src,
                                               uint32_t* __restrict__ d, int64_t ld_dst,
                                               int64_t rows_left, int64_t cols_left,
                                               u32x4* __restrict__ lds) {
  constexpr int MT = TM / 4, NT = TN / 4, P = MT * NT / 256;
  constexpr int RPP = 256 / NT, CPP = 256 / MT;
  static_assert(P * 256 == MT * NT && RPP * NT == 256 && CPP * MT == 256 && 4 * P * CPP == TN,
                "tile geometry");
  static_assert((MT & (MT - 1)) == 0, "the chunk swizzle needs a power-of-two row");
  const int t = threadIdx.x;
  const int mj = t % NT, mi0 = t / NT;
  u32x4 v[P][4];
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const int r = 4 * (mi0 + k * RPP), c = 4 * mj;
    if (kEdge && !(r < rows_left && c < cols_left)) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[k][q] = __builtin_nontemporal_load((const u32x4*)(s + (r + q) * ld_src + c));
  }
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const int mi = mi0 + k * RPP;
    const u32x4* x = v[k];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = 4 * mj + q;
      lds[c * MT + (mi ^ ((c >> 2) & (MT - 1)))] = u32x4{x[0][q], x[1][q], x[2][q], x[3][q]};
    }
  }
  __syncthreads();
  const int j = t % MT, c0 = t / MT;
#pragma unroll
  for (int k = 0; k < 4 * P; ++k) {
    const int c = c0 + k * CPP;
    if (kEdge && !(4 * j < rows_left && c < cols_left)) continue;
    __builtin_nontemporal_store(lds[c * MT + (j ^ ((c >> 2) & (MT - 1)))],
                                (u32x4*)(d + c * ld_dst + 4 * j));
  }
}

template <int TM, int TN>
__global__ __launch_bounds__(256) void transpose_lds_kernel(const uint32_t* __restrict__ src,
                                                           int64_t ld_src, uint32_t* __restrict__ dst,
                                                           int64_t ld_dst, int64_t M, int64_t N,
                                                           int tiles_m) {
  __shared__ u32x4 lds[TN * (TM / 4)];
  const int tn = blockIdx.x / tiles_m, tm = blockIdx.x - tn * tiles_m;
  // this block's tile of both layouts: the tile origins are scalars, the
  // inside-tile strides are (ld_src, 1) and (1, ld_dst)
  const int64_t blk[2] = {TM, TN};
  const View<2, int64_t> tS = tile_slice(tiled_divide(row_major<int64_t>(M, N, ld_src), blk), (int64_t)tm, (int64_t)tn);
  const View<2, int64_t> tD = tile_slice(tiled_divide(col_major<int64_t>(M, N, ld_dst), blk), (int64_t)tm, (int64_t)tn);
  const int64_t rows_left = M - (int64_t)tm * TM, cols_left = N - (int64_t)tn * TN;
  if (rows_left >= TM && cols_left >= TN)
    transpose_tile<TM, TN, false>(src + tS.offset, tS.layout.stride[0], dst + tD.offset,
                                  tD.layout.stride[1], rows_left, cols_left, lds);
  else
    transpose_tile<TM, TN, true>(src + tS.offset, tS.layout.stride[0], dst + tD.offset,
                                 tD.layout.stride[1], rows_left, cols_left, lds);
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
// Row-major to row-major: block (x, y) copies chunk x (256 vectors or
// elements, one per thread) of row y.  On a 16384^2 fp32 copy this 2-D grid
// measured 6.53-6.54 TB/s, against 6.41-6.43 with the row and chunk
// recovered from a 1-D block index by a 64-bit division, and 6.55-6.57 for a
// flat copy of the same contiguous bytes; one 16-byte vector per thread beat
// 2 to 8 vectors (5.9-6.2) and 16 (5.2).
template <typename V>
__global__ __launch_bounds__(256) void copy_rows_kernel(const V* __restrict__ src, int64_t ld_src,
                                                       V* __restrict__ dst, int64_t ld_dst,
                                                       int64_t row_len) {
  const int64_t row = blockIdx.y, i = (int64_t)blockIdx.x * 256 + threadIdx.x;
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
  if (chunks > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
  // rows in batches of at most 65535, the grid's y limit
  for (int64_t r0 = 0; r0 < M; r0 += 65535) {
    const int64_t rows = M - r0 < 65535 ? M - r0 : 65535;
    hipLaunchKernelGGL(copy_rows_kernel<V>, dim3((unsigned)chunks, (unsigned)rows), dim3(256), 0, s,
                       (const V*)src + r0 * ld_src, ld_src, (V*)dst + r0 * ld_dst, ld_dst, row_len);
    if (hipGetLastError() != hipSuccess) return TLA_ERR_HIP;
  }
  return TLA_OK;
}

}  // namespace

int transpose_dispatch(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t M,
                       int64_t N, int eb, hipStream_t s) {
  if (eb == 4 && M % 4 == 0 && N % 4 == 0 && ld_src % 4 == 0 && ld_dst % 4 == 0 && aligned16(src) &&
      aligned16(dst)) {
    // 256 x 64 block tiles through LDS: 256-byte runs per source row, 1 KiB
    // runs per destination column, tile rows fastest in launch order.  On a
    // 16384^2 fp32 transpose (GB/s, a streaming copy of the same bytes
    // 6516-6566): 256x64 6193-6232; 256x128 6083-6104; 512x64 6027-6053;
    // 1024x32 6117; 256x32 6079; 128x128 5504-5559; 64x256 5457-5819;
    // launched tile columns fastest, or with each XCD given a contiguous
    // run of tiles, 256x64 drops to 4631-5330.  The register-only form
    // (4x4 micro-tiles, 8 x 8 lanes, 128-byte runs both ways) peaked at
    // 5481 with 64 x 256 tiles.
    constexpr int TM = 256, TN = 64;
    const int64_t tm = (M + TM - 1) / TM, tn = (N + TN - 1) / TN;
    if (tm * tn > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((transpose_lds_kernel<TM, TN>), dim3((unsigned)(tm * tn)), dim3(256), 0, s,
                       (const uint32_t*)src, ld_src, (uint32_t*)dst, ld_dst, M, N, (int)tm);
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
