// gemm_common.hpp -- pieces shared by the GEMM kernel files: the launch
// parameters, the tile scheduler, the direct-to-LDS and register-staged slab
// loaders, the MFMA fragment loader and the fused epilogue.
//
//   D = act(alpha_eff * A.B + beta*C + bias),  fp32 accumulation.
//
// Operand roles.  Both LDS slabs hold rows of K (A by m, B by n).  The MFMA
// is issued with the B rows as its first operand and the A rows as its
// second, so its 32x32 result is D^T: each lane then owns four consecutive
// columns of one row of D, which the epilogue reads (C) and writes (D) as
// 8-byte vectors.
#pragma once

#include <type_traits>

#include "kernels.hpp"
#include "tla/copy.hpp"
#include "tla/layout.hpp"
#include "tla/mfma.hpp"

namespace tla {

// p.flags: C / D / bias rows allow aligned 4-element (8-byte for 16-bit)
// vectors; C / D rows (16-bit) allow aligned 16-byte vectors; C / D are
// row-major 16-bit matrices at an even address (any pitch).
enum : int { kCVec = 1, kDVec = 2, kBiasVec = 4, kC16 = 8, kD16 = 16, kC2 = 32, kD2 = 64 };

struct GemmParams {
  const uint8_t* A;
  const uint8_t* B;
  const uint8_t* C;
  uint8_t* D;
  const uint8_t* bias;
  // (row, k) strides of the A view (rows = m) and the B view (rows = n), in
  // elements; (m, n) strides of C and D.
  int64_t a_sr, a_sk, b_sr, b_sk, c_sm, c_sn, d_sm, d_sn;
  int M, N, K;
  int c_type, d_type, bias_type, act;
  float alpha, beta;
  int tiles_m, tiles_n;
  int flags;
  // implicit-GEMM convolution view of A (used by the kConv kernels only):
  // image H x W x C (NHWC), filter R x S, output P x Q, stride (u, v),
  // padding (ph, pw), dilation (dh, dw)
  int cH, cW, cC, cR, cS, cP, cQ, cu, cv, cph, cpw, cdh, cdw;
};

// The two-group 256 x 256 kernel of gemm_pingpong.hip for 16-bit or e4m3
// operands in the fast layout (both operands K-contiguous with 16-byte
// aligned rows, K a multiple of 16 bytes, each operand below 2 GiB); with
// `bt`, 16-bit operands whose B is N-contiguous instead (16-byte aligned
// rows, N a multiple of 8); with `at`, 16-bit operands whose A is
// M-contiguous (16-byte aligned columns, M a multiple of 8).
int launch_pingpong(const GemmParams& p, int a_type, hipStream_t stream, bool bt = false,
                    bool at = false);
const void* pingpong_kernel(int a_type);

// The four-wavefront kernel of gemm_general.hip.  launch_general: its
// register-staged form, 128 x 128 tiles, any order, pitch, alignment and
// ragged K (the operand views are read from p's strides).
// launch_two_stage_e4m3: its direct-to-LDS form for e4m3 in the fast layout,
// 256 x 256 (big) or 128 x 128 tiles.  launch_conv_general: the register-
// staged implicit-GEMM convolution (16-bit; p holds the convolution view).
// general_kernel / two_stage_e4m3_kernel: the kernels those launch for
// K-contiguous operands, for occupancy queries.
int launch_general(const GemmParams& p, int type, hipStream_t stream);
int launch_two_stage_e4m3(const GemmParams& p, bool big, hipStream_t stream);
int launch_conv_general(const GemmParams& p, int type, hipStream_t stream);
const void* general_kernel(int type);
const void* two_stage_e4m3_kernel(bool big);

namespace {

constexpr int kThreads = 256;  // four wavefronts

// LDS slab geometry for rows of kRowBytes bytes of K (a power of two between
// 32 and 128): kChunks 16-byte chunks per row and the XOR swizzle
// f(row) = (row / rows-per-256-bytes) mod kChunks, so the 16 rows a
// quarter-wave reads at one logical chunk cover the 16 distinct 16-byte
// bank groups of a 256-byte LDS window.
template <int kRowBytes>
struct Slab {
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kRowShift = kRowBytes == 128 ? 1 : (kRowBytes == 64 ? 2 : 3);
  using Swz = XorSwizzle<kChunks, kRowShift>;
};

// Workgroup barrier for LDS stages filled by direct copies.  __syncthreads()
// would put a workgroup release fence in front of the barrier, and that fence
// waits for every copy still in flight into LDS (vmcnt(0)) -- including the
// ones issued for later stages, which would drain the pipeline at every
// barrier.  Each wave instead waits for exactly the copies of the tile it
// needs (wait_vmcnt) and then meets the others here; the acquire fence keeps
// the LDS reads that follow from moving above the barrier.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// s_waitcnt with only the vector-memory counter bounded (gfx9 encoding:
// vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// ds_read_b64_tr_b16: four 16-bit elements per lane, transposed across each
// quarter-wave (lane j gets element j % 4 of the 8 bytes addressed by lanes
// 4 e + j / 4, e = 0..3).  The restrict-qualified parameter gives the read
// its own alias scope: without one the compiler makes the read wait for
// every direct HBM -> LDS copy in flight (vmcnt(0)), as it does not for
// plain LDS reads; the kernels order their copies and reads with explicit
// waits and barriers either way.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 ds_read_tr16(const uint8_t* __restrict__ p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

__device__ __forceinline__ lds_void_t* to_lds(void* p) { return (lds_void_t*)(p); }

// ---------------------------------------------------------- tile scheduler
// Workgroup b is dispatched to XCD b % 8.  Tile ids are handed out so that
// each XCD gets a contiguous run of them, and runs are ordered GROUP_M tile
// rows at a time (tile row fastest), so the workgroups sharing one XCD's L2
// work on a compact block of D and reuse each other's A and B slabs.
__device__ __forceinline__ void schedule(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int kXcds = 8, kGroupM = 4;
  const int total = tiles_m * tiles_n;
  int id = bid;
  if (total % kXcds == 0) id = (bid % kXcds) * (total / kXcds) + bid / kXcds;
  const int per_group = kGroupM * tiles_n;
  const int first_m = (id / per_group) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in = id % per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

// ------------------------------------------------------------ fast loader
// One k-tile slab of ROWS rows x kRowBytes bytes via direct global -> LDS
// copies.  The strip-mined map (ROWS x kChunks chunks, 256 threads, one chunk
// per access) puts thread t of iteration it at LDS slot t + 256*it, which is the
// lane-linear slot the DMA writes; the lane fetches the logical chunk that
// the swizzle assigns to that slot.
template <int ROWS, int kRowBytes>
__device__ __forceinline__ void dma_slab(const uint8_t* __restrict__ base, int64_t row_bytes,
                                         int row0, int rows_valid, int64_t kbyte0, uint8_t* slab,
                                         int tid) {
  using Swz = typename Slab<kRowBytes>::Swz;
  constexpr int kChunks = Slab<kRowBytes>::kChunks;
  constexpr StripMinedMap map(ROWS, kChunks, kThreads, 1, ROWS * kChunks / kThreads);
  static_assert(map.well_formed(), "slab thread map");
#pragma unroll
  for (int it = 0; it < map.I; ++it) {
    const int r = map.strided(tid, it);
    const int c = Swz::chunk(r, map.contiguous(tid, 0));
    const int gr = min(row0 + r, rows_valid - 1);
    const uint8_t* src = base + gr * row_bytes + kbyte0 + c * 16;
    uint8_t* dst = slab + map.index(tid & ~63, it, 0) * 16;  // wave-uniform
    __builtin_amdgcn_global_load_lds(src, to_lds(dst), 16, 0, 0);
  }
}

// Instruction `it` of dma_slab on its own, so a kernel can spread the copy
// of a slab between its matrix-core instructions.
template <int ROWS, int kRowBytes, int NT = kThreads>
__device__ __forceinline__ void dma_one(const uint8_t* __restrict__ base, int64_t row_bytes,
                                        int row0, int rows_valid, int64_t kbyte0, uint8_t* slab,
                                        int tid, int it) {
  using Swz = typename Slab<kRowBytes>::Swz;
  constexpr int kChunks = Slab<kRowBytes>::kChunks;
  constexpr StripMinedMap map(ROWS, kChunks, NT, 1, ROWS * kChunks / NT);
  const int r = map.strided(tid, it);
  const int c = Swz::chunk(r, map.contiguous(tid, 0));
  const int gr = min(row0 + r, rows_valid - 1);
  const uint8_t* src = base + gr * row_bytes + kbyte0 + c * 16;
  uint8_t* dst = slab + map.index(tid & ~63, it, 0) * 16;  // wave-uniform
  __builtin_amdgcn_global_load_lds(src, to_lds(dst), 16, 0, 0);
}

// --------------------------------------------------------- general loader
// 16 bytes from any byte address p through dword-aligned loads: the 16
// aligned bytes at or below p (lo) and the dword holding p + 15 (hi); the
// return value is p % 4.  Each dword read holds at least one of the 16
// requested bytes, so the reads never leave the pages those bytes live on.
// When p is dword-aligned, hi re-reads the last dword of lo.  The loads are
// only issued here: realign16 shifts the bytes into place once they are
// needed, so a register-staged copy does not wait for them early.
__device__ __forceinline__ uint32_t load16_split(const uint8_t* p, i32x4& lo, uint32_t& hi) {
  typedef int i32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
  const uint32_t sh = (uint32_t)(uintptr_t)p & 3u;
  const uint8_t* q = p - sh;
  lo = *(const i32x4_a4*)q;
  hi = *(const uint32_t*)(q + (sh ? 16 : 12));
  return sh;
}

// The 16 bytes load16_split fetched, funnel-shifted down by sh bytes
// (v_alignbyte_b32 takes the high dword first and reads only sh's low two
// bits); sh = 0 returns lo.
__device__ __forceinline__ i32x4 realign16(const i32x4& lo, uint32_t hi, uint32_t sh) {
  const uint32_t w0 = lo[0], w1 = lo[1], w2 = lo[2], w3 = lo[3];
  i32x4 r;
  r[0] = (int)__builtin_amdgcn_alignbyte(w1, w0, sh);
  r[1] = (int)__builtin_amdgcn_alignbyte(w2, w1, sh);
  r[2] = (int)__builtin_amdgcn_alignbyte(w3, w2, sh);
  r[3] = (int)__builtin_amdgcn_alignbyte(hi, w3, sh);
  return r;
}

// kCE = 16 / EB elements e = 0 .. kCE - 1 of a line, element e at
// p + min(i + e, last) * step: the ones with i + e < lim as loaded, the
// others zero.  Every address is clamped to element `last`, so all loads are
// issued unconditionally and stay inside the matrix.
template <int EB>
__device__ __forceinline__ i32x4 gather16(const uint8_t* p, int64_t step, int i, int lim,
                                          int last) {
  constexpr int kCE = 16 / EB;
  uint8_t bytes[16];
#pragma unroll
  for (int e = 0; e < kCE; ++e) {
    const uint8_t* q = p + (int64_t)min(i + e, last) * step;
    const bool ok = i + e < lim;
#pragma unroll
    for (int b = 0; b < EB; ++b) {
      const uint8_t x = q[b];
      bytes[e * EB + b] = ok ? x : 0;
    }
  }
  return __builtin_bit_cast(i32x4, bytes);
}

// Register-staged slab copy of an operand view (row, k) -> row*s_r +
// k*s_k, fixed at compile time to one of the two views the library builds:
// kKC (K-contiguous, s_k = 1) or row-contiguous (s_r = 1, an M- or
// N-contiguous matrix).  K-contiguous views use the row-contiguous thread
// map (consecutive lanes walk K) and move a tile inside K as whole 16-byte
// chunks through load16_split (load_whole), shifted into place by store();
// the last, ragged tile (load_edge) moves its chunks inside K the same way
// and the one that crosses K element by element, and the other view (the
// column-major map: consecutive lanes walk rows, so each element load
// coalesces) goes element by element.  Elements past K load as zero; rows
// past rows_valid repeat the last row (their products land in rows or
// columns of D that are never stored).  load_whole has no per-lane branch,
// so its loads stay in flight until store().
template <int ROWS, int EB, int kRowBytes, bool kKC>
struct RegSlab {
  using Swz = typename Slab<kRowBytes>::Swz;
  static constexpr int kChunks = Slab<kRowBytes>::kChunks;
  static constexpr int kI = ROWS * kChunks / kThreads;
  static constexpr int kCE = 16 / EB;  // elements per 16-byte chunk
  static constexpr int kTileK = kChunks * kCE;
  static_assert(kI <= 8, "byte shifts pack 4 bits per chunk");
  i32x4 v[kI];
  uint32_t hi[kI];
  uint32_t shifts;  // byte shift of chunk it in bits 4 it .. 4 it + 1

  static constexpr StripMinedMap map() {
    return StripMinedMap(ROWS, kChunks, kThreads, 1, kI, kKC ? 1 : 0);
  }

  // k0 .. k0 + kTileK - 1 inside K; s: the row stride in elements
  __device__ __forceinline__ void load_whole(const uint8_t* __restrict__ base, int64_t s, int row0,
                                             int rows_valid, int k0, int tid) {
    static_assert(kKC, "whole chunks along K");
    constexpr StripMinedMap m = map();
    static_assert(m.well_formed(), "slab thread map");
    shifts = 0;
#pragma unroll
    for (int it = 0; it < kI; ++it) {
      const int gr = min(row0 + m.row(tid, it, 0), rows_valid - 1);
      const uint8_t* p = base + (gr * s + (int64_t)(k0 + m.col(tid, it, 0) * kCE)) * EB;
      shifts |= load16_split(p, v[it], hi[it]) << (4 * it);
    }
  }

  // s: the row stride (kKC) or the k stride (otherwise), in elements.
  // Chunks past K are zero without a load; a K-contiguous chunk inside K
  // moves whole, the one that crosses K (and every chunk of the other view)
  // element by element.
  __device__ __forceinline__ void load_edge(const uint8_t* __restrict__ base, int64_t s, int row0,
                                            int rows_valid, int k0, int K, int tid) {
    constexpr StripMinedMap m = map();
    static_assert(m.well_formed(), "slab thread map");
    shifts = 0;
#pragma unroll
    for (int it = 0; it < kI; ++it) {
      const int gr = min(row0 + m.row(tid, it, 0), rows_valid - 1);
      const int gk = k0 + m.col(tid, it, 0) * kCE;
      const int64_t s_r = kKC ? s : 1, s_k = kKC ? 1 : s;
      const uint8_t* row = base + gr * s_r * EB;
      i32x4 x = {0, 0, 0, 0};
      uint32_t h = 0;
      if (gk < K) {
        if (kKC && gk + kCE <= K)
          shifts |= load16_split(row + (int64_t)gk * EB, x, h) << (4 * it);
        else
          x = gather16<EB>(row, s_k * EB, gk, K, K - 1);
      }
      v[it] = x;
      hi[it] = h;
    }
  }

  __device__ __forceinline__ void store(uint8_t* slab, int tid) const {
    constexpr StripMinedMap m = map();
#pragma unroll
    for (int it = 0; it < kI; ++it) {
      const int r = m.row(tid, it, 0), c = m.col(tid, it, 0);
      *(i32x4*)(slab + r * kRowBytes + Swz::chunk(r, c) * 16) =
          kKC ? realign16(v[it], hi[it], shifts >> (4 * it)) : v[it];
    }
  }
};

// N-contiguous 16-bit B (a row-major K x N matrix, pitch ld elements) for
// the register-staged kernel.  The slab is BK rows of k, each BN columns of
// n (2 BN bytes; 16-byte chunk c of row r stored at chunk c ^ 4 (r % 4)),
// and load_frag_nt reads it back with ds_read_b64_tr_b16.  Consecutive
// lanes walk the chunks of one k row, so a load instruction covers runs of
// whole rows; tiles inside K move whole chunks through load16_split
// (load_whole), the ragged k-tile chunk by chunk with rows past K zero and
// the chunk that crosses N element by element (load_edge).
template <int BN, int BK>
struct RegSlabNT {
  static constexpr int kRow = 2 * BN;
  static constexpr int kCh = kRow / 16;
  static constexpr int kI = BK * kCh / kThreads;
  static_assert(kI * kThreads == BK * kCh, "whole chunks per thread");
  static_assert(kCh >= 16 && kCh % 16 == 0, "the swizzle permutes chunks within 16");
  static_assert(kI <= 8, "byte shifts pack 4 bits per chunk");
  i32x4 v[kI];
  uint32_t hi[kI];
  uint32_t shifts;  // byte shift of chunk it in bits 4 it .. 4 it + 1

  // Rows k0 .. k0 + BK - 1 inside K, N >= 8.  A chunk that starts past N
  // reads columns N - 8 .. N - 1 instead and the chunk that crosses N reads
  // on past it: their columns past N only feed columns of D that are never
  // stored.  Reading past N stays inside the matrix while a row follows
  // (row k0 + BK - 1 below K - 1, or the tile inside N).
  __device__ __forceinline__ void load_whole(const uint8_t* __restrict__ base, int64_t ld, int n0,
                                             int N, int k0, int tid) {
    shifts = 0;
#pragma unroll
    for (int it = 0; it < kI; ++it) {
      const int sc = tid + kThreads * it, r = sc / kCh, c = sc % kCh;
      const int gn = n0 + 8 * c;
      const uint8_t* p = base + ((int64_t)(k0 + r) * ld + (gn < N ? gn : N - 8)) * 2;
      shifts |= load16_split(p, v[it], hi[it]) << (4 * it);
    }
  }

  // Chunks past K or N are zero without a load, chunks inside both move
  // whole, the chunk that crosses N element by element.
  __device__ __forceinline__ void load_edge(const uint8_t* __restrict__ base, int64_t ld, int n0,
                                            int N, int k0, int K, int tid) {
    shifts = 0;
#pragma unroll
    for (int it = 0; it < kI; ++it) {
      const int sc = tid + kThreads * it, r = sc / kCh, c = sc % kCh;
      const int gk = k0 + r, gn = n0 + 8 * c;
      i32x4 x = {0, 0, 0, 0};
      uint32_t h = 0;
      if (gk < K && gn < N) {
        const uint8_t* row = base + (int64_t)gk * ld * 2;
        if (gn + 8 <= N)
          shifts |= load16_split(row + (int64_t)gn * 2, x, h) << (4 * it);
        else
          x = gather16<2>(row, 2, gn, N, N - 1);
      }
      v[it] = x;
      hi[it] = h;
    }
  }

  __device__ __forceinline__ void store(uint8_t* slab, int tid) const {
#pragma unroll
    for (int it = 0; it < kI; ++it) {
      const int sc = tid + kThreads * it, r = sc / kCh, c = sc % kCh;
      *(i32x4*)(slab + r * kRow + (c ^ (4 * (r & 3))) * 16) =
          realign16(v[it], hi[it], shifts >> (4 * it));
    }
  }
};

// The B fragment of 32x32x16 MFMA k-step ks for columns col0 .. col0 + 31
// of a RegSlabNT slab (rows of kRow bytes): lane l gets column col0 + l % 32,
// k = 16 ks + 8 (l / 32) .. + 7, as two ds_read_b64_tr_b16.  In a
// quarter-wave the instruction hands lane j element e of the 8 bytes that
// lane 4 e + j / 4 addresses, at position j % 4, so lane a of the quarter
// addresses row k0 + a / 4, columns n0 + 4 (a % 4) .. + 3, and lane j
// receives B[k0 .. k0 + 3][n0 + j].  Rows k0 .. k0 + 3 of one 32-column
// half-wave land on 16 distinct 16-byte bank groups under the swizzle.
template <int kRow>
__device__ __forceinline__ i32x4 load_frag_nt(const uint8_t* slab, int col0, int ks, int lane) {
  typedef int s32x2 __attribute__((ext_vector_type(2)));
  const int qw = lane >> 4, a4 = lane & 15;
  const int n = col0 + 16 * (qw & 1) + 4 * (a4 & 3);
  s32x2 h[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int k = 16 * ks + 8 * (qw >> 1) + 4 * hh + (a4 >> 2);
    h[hh] = __builtin_bit_cast(
        s32x2, ds_read_tr16(slab + k * kRow + ((n >> 3) ^ (4 * (k & 3))) * 16 + (n & 7) * 2));
  }
  return i32x4{h[0][0], h[0][1], h[1][0], h[1][1]};
}

// ---------------------------------------------- implicit-GEMM A loader
// The A operand of a convolution seen as a GEMM (the implicit GEMM of the
// PitchLinearStripminedThreadMap walk-through, section 5.2): row m is the
// output pixel (n, p, q) = (m / PQ, m / Q mod P, m mod Q), column k the
// filter position and channel (r, s, c) = (k / (S C), k / C mod S, k mod C),
// and the element is x[n, p u - ph + r dh, q v - pw + s dw, c] -- zero outside
// the image.  The slab is walked with the same row-contiguous strip-mined
// map as a K-contiguous operand; when C is a multiple of the vector width
// (and the image is 16-byte aligned) a 16-byte chunk never straddles a
// filter position, so one bounds check covers it.
template <int ROWS, int EB, int kRowBytes>
struct ConvSlab : RegSlab<ROWS, EB, kRowBytes, true> {
  using Base = RegSlab<ROWS, EB, kRowBytes, true>;

  __device__ __forceinline__ const uint8_t* at(const GemmParams& p, int n, int h0, int w0,
                                               int k) const {
    const int c = k % p.cC, rs = k / p.cC;
    const int r = rs / p.cS, s = rs - r * p.cS;
    const int h = h0 + r * p.cdh, w = w0 + s * p.cdw;
    if (h < 0 || h >= p.cH || w < 0 || w >= p.cW) return nullptr;
    return p.A + ((((int64_t)n * p.cH + h) * p.cW + w) * p.cC + c) * EB;
  }

  __device__ __forceinline__ void load_conv(const GemmParams& p, int row0, int k0, bool vec_ok,
                                            int tid) {
    constexpr StripMinedMap kmap(ROWS, Base::kChunks, kThreads, 1, Base::kI, 1);
    constexpr int kCE = Base::kCE;
    const int PQ = p.cP * p.cQ;
    this->shifts = 0;  // whole chunks are loaded aligned or element by element
#pragma unroll
    for (int it = 0; it < Base::kI; ++it) {
      const int m = row0 + kmap.row(tid, it, 0);
      const int k = k0 + kmap.col(tid, it, 0) * kCE;
      i32x4 x = {0, 0, 0, 0};
      if (m < p.M) {
        const int n = m / PQ, pq = m - n * PQ, pp = pq / p.cQ, qq = pq - pp * p.cQ;
        const int h0 = pp * p.cu - p.cph, w0 = qq * p.cv - p.cpw;
        if (vec_ok && k + kCE <= p.K) {
          const uint8_t* src = at(p, n, h0, w0, k);
          if (src) x = *(const i32x4*)src;
        } else {
          uint8_t bytes[16] = {};
#pragma unroll
          for (int e = 0; e < kCE; ++e) {
            if (k + e < p.K) {
              const uint8_t* src = at(p, n, h0, w0, k + e);
              if (src) {
#pragma unroll
                for (int b = 0; b < EB; ++b) bytes[e * EB + b] = src[b];
              }
            }
          }
          x = __builtin_bit_cast(i32x4, bytes);
        }
      }
      this->v[it] = x;
      this->hi[it] = 0;
    }
  }
};

// ------------------------------------------------------- fragment loader
// Lane l's operand fragment for MFMA k-step ks: row `row` of the slab, the
// (l/32)-th kLaneBytes-wide half of the step's K bytes.
template <int kCode, int kRowBytes>
__device__ __forceinline__ typename MfmaAtom<kCode>::Frag load_frag(const uint8_t* slab, int row,
                                                                   int ks, int lane) {
  using Atom = MfmaAtom<kCode>;
  using Swz = typename Slab<kRowBytes>::Swz;
  constexpr int kStepBytes = Atom::kK * elem_bytes(kCode);
  const int c0 = (ks * kStepBytes + (lane >> 5) * Atom::kLaneBytes) / 16;
  const uint8_t* rowp = slab + row * kRowBytes;
  if constexpr (Atom::kLaneBytes == 16) {
    return *(const i32x4*)(rowp + Swz::chunk(row, c0) * 16);
  } else {
    i32x4 lo = *(const i32x4*)(rowp + Swz::chunk(row, c0) * 16);
    i32x4 hi = *(const i32x4*)(rowp + Swz::chunk(row, c0 + 1) * 16);
    return typename Atom::Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// ---------------------------------------------------------------- epilogue
__device__ __forceinline__ float load_elem(const uint8_t* p, int type, int64_t idx) {
  if (type == kF32) return ((const float*)p)[idx];
  const uint16_t h = ((const uint16_t*)p)[idx];
  if (type == kBF16) return __builtin_bit_cast(float, (uint32_t)h << 16);
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t to_bits(float v, int type) {
  if (type == kBF16) return __builtin_bit_cast(uint16_t, (__bf16)v);
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

__device__ __forceinline__ void load4(const uint8_t* p, int type, int64_t idx, float (&x)[4]) {
  if (type == kF32) {
    const f32x4 v = *(const f32x4*)((const float*)p + idx);
    x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
  } else {
    const uint2 u = *(const uint2*)((const uint16_t*)p + idx);
    const uint32_t w[4] = {u.x & 0xFFFFu, u.x >> 16, u.y & 0xFFFFu, u.y >> 16};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      x[q] = (type == kBF16) ? __builtin_bit_cast(float, w[q] << 16)
                             : (float)__builtin_bit_cast(_Float16, (uint16_t)w[q]);
  }
}

// GELU(y) = y * Phi(y), Phi the standard normal distribution function, in
// erfc form: with h = erfc(a) / 2, a = |y| / sqrt(2), Phi(y) is 1 - h for
// y >= 0 and h for y < 0, so GELU(y) = max(y, 0) - |y| h.
// erfc(a) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^(-a^2), t = 1 / (1 + p a),
// is formula 7.1.26 of Abramowitz and Stegun, Handbook of Mathematical
// Functions (|error| <= 1.5e-7).  Here the coefficients are halved and the
// argument is b = a sqrt(log2 e), so that e^(-a^2) = 2^(-b^2) and
// p a = (p / sqrt(log2 e)) b.  Branch-free, 14 vector operations (two of
// them the hardware reciprocal and exp2) against about 30 with a divergent
// branch for 1 + erf(y / sqrt 2); |Phi - exact| <= 3e-7 in fp32, the same
// as the erf form.  |y| is clamped to the largest float so that
// GELU(+inf) = +inf and GELU(-inf) = 0.  The epilogue applies it to every
// accumulator, 128 per lane per tile.
__device__ __forceinline__ float gelu(float y) {
  const float ay = fminf(fabsf(y), 3.40282347e38f);
  const float b = ay * 0.8493218003f;                  // |y| sqrt(log2(e) / 2)
  const float t = __builtin_amdgcn_rcpf(fmaf(0.2727374809f, b, 1.0f));
  float q = fmaf(t, 0.5307027145f, -0.7265760135f);
  q = fmaf(t, q, 0.7107068705f);
  q = fmaf(t, q, -0.142248368f);
  q = fmaf(t, q, 0.127414796f);
  const float h = q * t * __builtin_amdgcn_exp2f(b * -b);
  return fmaf(-ay, h, fmaxf(y, 0.f));
}

__device__ __forceinline__ float activate(float y, int act) {
  if (act == TLA_ACT_RELU) return y > 0.f ? y : 0.f;
  if (act == TLA_ACT_GELU) return gelu(y);
  return y;
}

// Four consecutive columns n..n+3 of row m.
__device__ __forceinline__ void epilogue4(const GemmParams& p, int m, int n, const float (&acc)[4]) {
  if (m >= p.M || n >= p.N) return;
  const bool full = n + 3 < p.N;
  float y[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) y[q] = p.alpha * acc[q];
  if (p.beta != 0.f) {
    float c[4] = {0.f, 0.f, 0.f, 0.f};
    if (full && (p.flags & kCVec)) {
      load4(p.C, p.c_type, m * p.c_sm + (int64_t)n, c);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (n + q < p.N) c[q] = load_elem(p.C, p.c_type, m * p.c_sm + (int64_t)(n + q) * p.c_sn);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] += p.beta * c[q];
  }
  if (p.bias) {
    float b[4] = {0.f, 0.f, 0.f, 0.f};
    if (full && (p.flags & kBiasVec)) {
      load4(p.bias, p.bias_type, n, b);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (n + q < p.N) b[q] = load_elem(p.bias, p.bias_type, n + q);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] += b[q];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) y[q] = activate(y[q], p.act);
  uint16_t* D = (uint16_t*)p.D;
  if (full && (p.flags & kDVec)) {
    uint2 u;
    u.x = (uint32_t)to_bits(y[0], p.d_type) | ((uint32_t)to_bits(y[1], p.d_type) << 16);
    u.y = (uint32_t)to_bits(y[2], p.d_type) | ((uint32_t)to_bits(y[3], p.d_type) << 16);
    *(uint2*)(D + m * p.d_sm + n) = u;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (n + q < p.N) D[m * p.d_sm + (int64_t)(n + q) * p.d_sn] = to_bits(y[q], p.d_type);
  }
}

// ------------------------------------------- specialised full-tile epilogue
// The two fast epilogue paths below are compiled per activation, per
// 16-bit type (shared by C, bias and D) and with or without C, so the
// per-element work is straight-line code: one fma for alpha*acc + bias,
// one widening and one fma for beta*C, the activation and a packed
// conversion.  The low and high halves of a packed pair widen in one
// operation each.
template <bool kBf16>
__device__ __forceinline__ float widen_lo(uint32_t w) {
  if constexpr (kBf16) return __builtin_bit_cast(float, w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
template <bool kBf16>
__device__ __forceinline__ float widen_hi(uint32_t w) {
  if constexpr (kBf16) return __builtin_bit_cast(float, w & 0xFFFF0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

template <int kAct>
__device__ __forceinline__ float act_t(float y) {
  if constexpr (kAct == TLA_ACT_RELU) return y > 0.f ? y : 0.f;
  if constexpr (kAct == TLA_ACT_GELU) return gelu(y);
  return y;
}

template <bool kBf16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (kBf16)
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
  else
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// y = act(alpha*acc + bias + beta*c) for the four values of group g of tile
// (i, j); c and bias arrive as packed 16-bit pairs (bias zero bits when
// there is none).
template <int kAct, bool kBf16, bool kHasC>
__device__ __forceinline__ uint2 epi_group(const f32x16& acc, int g, uint2 c, uint2 b, float alpha,
                                           float beta) {
  const float bias[4] = {widen_lo<kBf16>(b.x), widen_hi<kBf16>(b.x), widen_lo<kBf16>(b.y),
                         widen_hi<kBf16>(b.y)};
  float y[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) y[q] = fmaf(alpha, acc[4 * g + q], bias[q]);
  if constexpr (kHasC) {
    y[0] = fmaf(beta, widen_lo<kBf16>(c.x), y[0]);
    y[1] = fmaf(beta, widen_hi<kBf16>(c.x), y[1]);
    y[2] = fmaf(beta, widen_lo<kBf16>(c.y), y[2]);
    y[3] = fmaf(beta, widen_hi<kBf16>(c.y), y[3]);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) y[q] = act_t<kAct>(y[q]);
  return uint2{pack2<kBf16>(y[0], y[1]), pack2<kBf16>(y[2], y[3])};
}

// This lane's 16-bit bias values for its column groups, all loads issued
// before any is used (zero bits when there is no bias).
// cols: the wave tile's columns inside D; a group past them reads the
// aligned group that holds the last column instead (bias is 8-byte aligned,
// so that read stays on the last element's page), feeding only columns of D
// that are never stored.
template <int FN>
__device__ __forceinline__ void load_bias16(const GemmParams& p, int n_base, int half,
                                            uint2 (&braw)[FN][4], int cols = 32 * FN) {
  static_for<FN>([&](auto j) { static_for<4>([&](auto g) { braw[j][g] = uint2{0u, 0u}; }); });
  if (p.bias) {
    const uint16_t* b = (const uint16_t*)p.bias + n_base;
    const int last4 = (cols - 1) & ~3;
    static_for<FN>([&](auto j) {
      static_for<4>([&](auto g) {
        braw[j][g] = *(const uint2*)(b + min(32 * j + 8 * g + 4 * half, last4));
      });
    });
  }
}

// Full wave tile through LDS.  In the MFMA result layout a lane holds four
// consecutive columns of one row, so a direct global access touches 32 rows
// 16 bytes at a time.  Instead the wave copies its C sub-tile (WM rows of
// 64*FN bytes) into its own LDS region with whole-row direct copies, applies
// the epilogue reading C there in the MFMA layout, writes the 16-bit result
// back in place and stores D from LDS as whole rows.  The region's 16-byte
// chunks are XOR-swizzled by row so that the lane-per-row accesses of one
// instruction fall into distinct LDS banks.
template <int kAct, bool kDBf16, bool kHasC, int FM, int FN>
__device__ __forceinline__ void epilogue_lds(const GemmParams& p, int m_base, int n_base, int lane,
                                             const f32x16 (&acc)[FM][FN], uint8_t* region) {
  constexpr int kRowB = 64 * FN, kCh = kRowB / 16, kRowsPerKiB = 1024 / kRowB;
  static_assert(kCh == 4 || kCh == 8 || kCh == 16, "row width");
  constexpr int kIters = 32 * FM * kRowB / 1024;
  auto swz = [](int r, int c) { return c ^ ((r / (16 / kCh)) & (kCh - 1)); };
  const int row = lane & 31, half = lane >> 5;
  const int rr = lane / kCh, cs = lane % kCh;  // row-wise view of one KiB
  if constexpr (kHasC) {
    const uint8_t* C = p.C + ((int64_t)m_base * p.c_sm + n_base) * 2;
    static_for<kIters>([&](auto t) {
      const int r = kRowsPerKiB * t + rr;
      const uint8_t* src = C + (int64_t)r * p.c_sm * 2 + swz(r, cs) * 16;
      __builtin_amdgcn_global_load_lds(src, to_lds(region + t * 1024), 16, 0, 0);
    });
  }
  uint2 braw[FN][4];
  load_bias16<FN>(p, n_base, half, braw);
  wait_vmcnt<0>();  // this wave's C copies have landed in its region
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  static_for<FM>([&](auto i) {
    static_for<FN>([&](auto j) {
      static_for<4>([&](auto g) {
        const int r = 32 * i + row;
        uint8_t* slot = region + r * kRowB + swz(r, 4 * j + g) * 16 + 8 * half;
        const uint2 c = kHasC ? *(const uint2*)slot : uint2{0u, 0u};
        *(uint2*)slot = epi_group<kAct, kDBf16, kHasC>(acc[i][j], g, c, braw[j][g], p.alpha, p.beta);
      });
    });
  });
  uint8_t* D = p.D + ((int64_t)m_base * p.d_sm + n_base) * 2;
  static_for<kIters>([&](auto t) {
    const int r = kRowsPerKiB * t + rr;
    const i32x4 v = *(const i32x4*)(region + t * 1024 + lane * 16);
    *(i32x4*)(D + (int64_t)r * p.d_sm * 2 + swz(r, cs) * 16) = v;
  });
}

// 16 bytes to an even address p: one 16-byte store when p is dword-aligned,
// else a 2-byte, a 12-byte (dword-aligned) and a 2-byte store, so no byte
// outside [p, p + 16) is written.
__device__ __forceinline__ void store16_even(uint8_t* p, const i32x4& v) {
  typedef int i32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
  typedef int i32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));
  if (((uint32_t)(uintptr_t)p & 2u) == 0) {
    *(i32x4_a4*)p = v;
  } else {
    const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
    i32x3_a4 mid;
    mid[0] = (int)__builtin_amdgcn_alignbyte(w1, w0, 2);
    mid[1] = (int)__builtin_amdgcn_alignbyte(w2, w1, 2);
    mid[2] = (int)__builtin_amdgcn_alignbyte(w3, w2, 2);
    *(uint16_t*)p = (uint16_t)w0;
    *(i32x3_a4*)(p + 2) = mid;
    *(uint16_t*)(p + 14) = (uint16_t)(w3 >> 16);
  }
}

// epilogue_lds for C and D rows at any even address (any pitch): the wave
// reads its C sub-tile row by row with realigned 16-byte loads
// (load16_split) and writes it into its region in the same swizzled layout,
// and stores D row by row through store16_even.  Consecutive lanes cover a
// row's consecutive chunks, so each access instruction spans whole rows
// instead of 32 rows 8 bytes apart.  Only the first `rows` rows and `cols`
// columns of the wave tile are in D: C reads of the other rows repeat the
// last one and they store nothing; in a tile that ends inside N the chunk
// that crosses N moves element by element and chunks past it are skipped.
template <int kAct, bool kDBf16, bool kHasC, int FM, int FN>
__device__ __forceinline__ void epilogue_lds_any(const GemmParams& p, int m_base, int n_base,
                                                 int lane, const f32x16 (&acc)[FM][FN],
                                                 uint8_t* region, int rows, int cols) {
  constexpr int kRowB = 64 * FN, kCh = kRowB / 16, kRowsPerKiB = 1024 / kRowB;
  static_assert(kCh == 4 || kCh == 8 || kCh == 16, "row width");
  constexpr int kIters = 32 * FM * kRowB / 1024;
  static_assert(kIters <= 8, "byte shifts pack 4 bits per row chunk");
  auto swz = [](int r, int c) { return c ^ ((r / (16 / kCh)) & (kCh - 1)); };
  const int row = lane & 31, half = lane >> 5;
  const int rr = lane / kCh, cs = lane % kCh;  // row-wise view of one KiB
  const bool all_cols = cols == 32 * FN;
  if constexpr (kHasC) {
    const uint8_t* C = p.C + ((int64_t)m_base * p.c_sm + n_base) * 2;
    if (all_cols) {
      i32x4 lo[kIters];
      uint32_t hi[kIters], shifts = 0;
      static_for<kIters>([&](auto t) {
        const int r = kRowsPerKiB * t + rr;
        const int rc = min(r, rows - 1);
        shifts |= load16_split(C + (int64_t)rc * p.c_sm * 2 + swz(r, cs) * 16, lo[t], hi[t])
                  << (4 * t);
      });
      static_for<kIters>([&](auto t) {
        *(i32x4*)(region + t * 1024 + lane * 16) = realign16(lo[t], hi[t], shifts >> (4 * t));
      });
    } else {
      static_for<kIters>([&](auto t) {
        const int r = kRowsPerKiB * t + rr;
        const int c0 = 8 * swz(r, cs);  // first column of the chunk
        const uint8_t* rowp = C + (int64_t)min(r, rows - 1) * p.c_sm * 2;
        i32x4 x = {0, 0, 0, 0};
        if (c0 + 8 <= cols) {
          i32x4 lo;
          uint32_t hi;
          const uint32_t sh = load16_split(rowp + c0 * 2, lo, hi);
          x = realign16(lo, hi, sh);
        } else if (c0 < cols) {
          x = gather16<2>(rowp, 2, c0, cols, cols - 1);
        }
        *(i32x4*)(region + t * 1024 + lane * 16) = x;
      });
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
  uint2 braw[FN][4];
  load_bias16<FN>(p, n_base, half, braw, cols);
  static_for<FM>([&](auto i) {
    static_for<FN>([&](auto j) {
      static_for<4>([&](auto g) {
        const int r = 32 * i + row;
        uint8_t* slot = region + r * kRowB + swz(r, 4 * j + g) * 16 + 8 * half;
        const uint2 c = kHasC ? *(const uint2*)slot : uint2{0u, 0u};
        *(uint2*)slot = epi_group<kAct, kDBf16, kHasC>(acc[i][j], g, c, braw[j][g], p.alpha, p.beta);
      });
    });
  });
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  uint8_t* D = p.D + ((int64_t)m_base * p.d_sm + n_base) * 2;
  static_for<kIters>([&](auto t) {
    const int r = kRowsPerKiB * t + rr;
    const int c0 = 8 * swz(r, cs);
    const i32x4 v = *(const i32x4*)(region + t * 1024 + lane * 16);
    uint8_t* dst = D + (int64_t)r * p.d_sm * 2 + c0 * 2;
    if (r < rows) {
      if (c0 + 8 <= cols) {
        store16_even(dst, v);
      } else if (c0 < cols) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e < cols) ((uint16_t*)dst)[e] = (uint16_t)((uint32_t)v[e >> 1] >> (16 * (e & 1)));
      }
    }
  });
}

// Full wave tile straight from and to global memory with 8-byte vectors;
// all C and bias loads are issued before the arithmetic.
template <int kAct, bool kDBf16, bool kHasC, int FM, int FN>
__device__ __forceinline__ void epilogue_direct(const GemmParams& p, int m_base, int n_base, int lane,
                                                const f32x16 (&acc)[FM][FN]) {
  const int row = lane & 31, half = lane >> 5;
  uint2 c[FM][FN][4];
  if constexpr (kHasC) {
    const uint16_t* C = (const uint16_t*)p.C;
    static_for<FM>([&](auto i) {
      static_for<FN>([&](auto j) {
        static_for<4>([&](auto g) {
          c[i][j][g] = *(const uint2*)(C + (int64_t)(m_base + 32 * i + row) * p.c_sm + n_base + 32 * j +
                                       8 * g + 4 * half);
        });
      });
    });
  } else {
    static_for<FM>([&](auto i) {
      static_for<FN>([&](auto j) { static_for<4>([&](auto g) { c[i][j][g] = uint2{0u, 0u}; }); });
    });
  }
  uint2 braw[FN][4];
  load_bias16<FN>(p, n_base, half, braw);
  uint16_t* D = (uint16_t*)p.D;
  static_for<FM>([&](auto i) {
    static_for<FN>([&](auto j) {
      static_for<4>([&](auto g) {
        *(uint2*)(D + (int64_t)(m_base + 32 * i + row) * p.d_sm + n_base + 32 * j + 8 * g + 4 * half) =
            epi_group<kAct, kDBf16, kHasC>(acc[i][j], g, c[i][j][g], braw[j][g], p.alpha, p.beta);
      });
    });
  });
}

// kForm: 0 direct, 1 LDS with 16-byte aligned rows, 2 LDS with rows at any
// even address
template <int kForm, int kAct, bool kDBf16, int FM, int FN>
__device__ __forceinline__ void epilogue_fast(const GemmParams& p, int m_base, int n_base, int lane,
                                              const f32x16 (&acc)[FM][FN], uint8_t* region,
                                              int rows, int cols) {
  const bool has_c = p.beta != 0.f;
  if constexpr (kForm == 1) {
    if (has_c) epilogue_lds<kAct, kDBf16, true, FM, FN>(p, m_base, n_base, lane, acc, region);
    else epilogue_lds<kAct, kDBf16, false, FM, FN>(p, m_base, n_base, lane, acc, region);
  } else if constexpr (kForm == 2) {
    if (has_c)
      epilogue_lds_any<kAct, kDBf16, true, FM, FN>(p, m_base, n_base, lane, acc, region, rows,
                                                   cols);
    else
      epilogue_lds_any<kAct, kDBf16, false, FM, FN>(p, m_base, n_base, lane, acc, region, rows,
                                                    cols);
  } else {
    if (has_c) epilogue_direct<kAct, kDBf16, true, FM, FN>(p, m_base, n_base, lane, acc);
    else epilogue_direct<kAct, kDBf16, false, FM, FN>(p, m_base, n_base, lane, acc);
  }
}

// rows, cols: the wave tile's rows and columns inside D (kForm 2 only; the
// others take whole tiles)
template <int kForm, int FM, int FN>
__device__ __forceinline__ void epilogue_switch(const GemmParams& p, int m_base, int n_base, int lane,
                                                const f32x16 (&acc)[FM][FN], uint8_t* region,
                                                int rows = 32 * FM, int cols = 32 * FN) {
  const bool dbf = p.d_type == kBF16;
  auto run = [&](auto act) {
    constexpr int kAct = decltype(act)::value;
    if (dbf) epilogue_fast<kForm, kAct, true>(p, m_base, n_base, lane, acc, region, rows, cols);
    else epilogue_fast<kForm, kAct, false>(p, m_base, n_base, lane, acc, region, rows, cols);
  };
  switch (p.act) {
    case TLA_ACT_RELU: run(std::integral_constant<int, TLA_ACT_RELU>{}); break;
    case TLA_ACT_GELU: run(std::integral_constant<int, TLA_ACT_GELU>{}); break;
    default: run(std::integral_constant<int, TLA_ACT_NONE>{}); break;
  }
}

// The epilogue of one wavefront's FM x FN grid of 32x32 accumulator tiles,
// rows m_base + 32i + lane%32, column groups n_base + 32j + 8g + 4(lane/32).
// `region` is this wave's 32*FM x 64*FN-byte piece of LDS, free for reuse
// (the caller has synchronised the workgroup after its last LDS read), or
// null.  A wave tile inside D whose C (if any) and bias (if any) have D's
// 16-bit type takes the LDS path when C and D rows allow 16-byte vectors,
// else the direct path with 8-byte vectors, else (kAny, row-major C and D
// at even addresses, any pitch) the LDS path with realigned row accesses,
// which (kAny) also takes wave tiles that end inside M, or inside N with
// at least half their columns in D (narrower ones spend less in epilogue4,
// whose groups past N return at once); anything else (other edge tiles,
// fp32 or mixed-type C or bias, column-major C or D) goes group by group
// through the predicated epilogue4.
template <int FM, int FN, bool kAny = false>
__device__ __forceinline__ void epilogue_tiles(const GemmParams& p, int m_base, int n_base, int lane,
                                               const f32x16 (&acc)[FM][FN], uint8_t* region) {
  const bool full = m_base + 32 * FM <= p.M && n_base + 32 * FN <= p.N;
  const bool b_ok = !p.bias || ((p.flags & kBiasVec) && p.bias_type == p.d_type);
  const bool c16 = p.c_type == p.d_type;
  if (full && b_ok && region && (p.flags & kD16) && (p.beta == 0.f || (c16 && (p.flags & kC16)))) {
    epilogue_switch<1, FM, FN>(p, m_base, n_base, lane, acc, region);
  } else if (full && b_ok && (p.flags & kDVec) && (p.beta == 0.f || (c16 && (p.flags & kCVec)))) {
    epilogue_switch<0, FM, FN>(p, m_base, n_base, lane, acc, region);
  } else if (kAny && m_base < p.M && p.N - n_base >= 16 * FN && b_ok && region &&
             (p.flags & kD2) && (p.beta == 0.f || (c16 && (p.flags & kC2)))) {
    if constexpr (kAny)
      epilogue_switch<2, FM, FN>(p, m_base, n_base, lane, acc, region, min(32 * FM, p.M - m_base),
                                 min(32 * FN, p.N - n_base));
  } else {
    static_for<FM>([&](auto i) {
      const int m = m_base + 32 * i + mfma32_acc_col(lane, 0);
      static_for<FN>([&](auto j) {
        static_for<4>([&](auto g) {
          const int n = n_base + 32 * j + mfma32_acc_row(lane, 4 * g);
          const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                              acc[i][j][4 * g + 3]};
          epilogue4(p, m, n, v);
        });
      });
    });
  }
}

// ------------------------------------------------------------- fast kernel
// 16 bytes per lane from base + voffset + soffset into LDS, landing
// lane-linearly from the wave-uniform address `lds`: a raw buffer load whose
// per-lane 32-bit offset and uniform offset stay separate registers, so the
// loop spends no vector instructions on copy addresses.  Every offset the
// kernel forms is below 2^31 (checked by the host).
// `records` bounds the buffer: a lane whose offset lies past it reads zeros
// (the raw buffer range check) and touches no memory.
__device__ __forceinline__ void dma16_buf(const uint8_t* base, uint32_t voffset, uint32_t soffset,
                                          uint8_t* lds, int records = 0x7FFFFFFF) {
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, records, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voffset,
                                           soffset, 0, 0);
#endif
}

bool aligned(const void* p, int64_t bytes) { return ((uintptr_t)p % (uintptr_t)bytes) == 0; }

void set_grid(GemmParams& p, int BM, int BN, int64_t* grid) {
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  *grid = (int64_t)p.tiles_m * p.tiles_n;
}

}  // namespace
}  // namespace tla
