// gemm.hip -- hierarchically tiled GEMM with a fused epilogue for gfx950.
//
//   D = act(alpha_eff * A.B + beta*C + bias),  fp32 accumulation.
//
// Three levels of tiling, as in "CUTLASS / CuTe 主线" (hpc.payai.win/cutlass),
// section 一: a workgroup owns a BM x BN tile of D (the block tile), each of
// its four 64-lane wavefronts a (BM/2) x (BN/2) quarter (the wave tile), and
// each 32x32 MFMA instruction a 32x32 piece of that (the instruction tile).
// The K loop (section 二's mainloop: global -> shared -> register) moves one
// 128-byte-wide K slab of A and of B per step into LDS (64 bf16/fp16 or 128
// e4m3 per row), double-buffered so the next slab streams in while the
// current one feeds the matrix cores (section 四: pipeline stages hide global
// latency).  The epilogue applies alpha, beta*C, bias and the activation to
// the fp32 accumulators in registers and stores D once (section 四: fuse
// before the store); for whole tiles the freed LDS stages turn C and D into
// whole-row transfers (see epilogue_lds).
//
// Operand roles.  Both LDS slabs hold rows of K (A by m, B by n).  The MFMA
// is issued with the B rows as its first operand and the A rows as its
// second, so its 32x32 result is D^T: each lane then owns four consecutive
// columns of one row of D, which the epilogue reads (C) and writes (D) as
// 8-byte vectors.
//
// Two load paths feed the same LDS layout:
//   fast    both operands K-contiguous, 16-byte aligned rows, K a multiple of
//           the slab width: each lane issues global_load_lds_dwordx4, a
//           direct HBM -> LDS copy that lands lane-linearly; the LDS XOR
//           swizzle is applied by permuting which global chunk each lane
//           fetches.  Rows past M or N are clamped to the last real row (their
//           results are never stored), so the loop carries no predicates.
//   general any order, pitch or alignment, ragged K: registers staged through
//           a strip-mined thread map with per-element predicates; elements
//           outside the matrix load as zero.
#include <type_traits>

#include "kernels.hpp"
#include "tla/copy.hpp"
#include "tla/layout.hpp"
#include "tla/mfma.hpp"

namespace tla {
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

// p.flags: C / D / bias rows allow aligned 4-element (8-byte for 16-bit)
// vectors; C / D rows (16-bit) allow aligned 16-byte vectors.
enum : int { kCVec = 1, kDVec = 2, kBiasVec = 4, kC16 = 8, kD16 = 16 };

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

typedef __attribute__((address_space(3))) void lds_void_t;

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
// Element-predicated, register-staged slab copy for any operand view
// (row, k) -> row*s_r + k*s_k.  K-contiguous views use the row-contiguous
// thread map (consecutive lanes walk K); the others use the column-major
// variant (consecutive lanes walk rows, so each element load coalesces).
template <int ROWS, int EB, int kRowBytes>
struct RegSlab {
  using Swz = typename Slab<kRowBytes>::Swz;
  static constexpr int kChunks = Slab<kRowBytes>::kChunks;
  static constexpr int kI = ROWS * kChunks / kThreads;
  static constexpr int kCE = 16 / EB;  // elements per 16-byte chunk
  i32x4 v[kI];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ base, int64_t s_r, int64_t s_k,
                                       int row0, int rows_valid, int k0, int K, bool vec_ok,
                                       int tid) {
    constexpr StripMinedMap kmap(ROWS, kChunks, kThreads, 1, kI, 1);
    constexpr StripMinedMap rmap(ROWS, kChunks, kThreads, 1, kI, 0);
    static_assert(kmap.well_formed() && rmap.well_formed(), "slab thread maps");
    const bool kcontig = (s_k == 1);
#pragma unroll
    for (int it = 0; it < kI; ++it) {
      const int r = kcontig ? kmap.row(tid, it, 0) : rmap.row(tid, it, 0);
      const int c = kcontig ? kmap.col(tid, it, 0) : rmap.col(tid, it, 0);
      const int gr = row0 + r;
      const int gk = k0 + c * kCE;
      i32x4 x = {0, 0, 0, 0};
      if (gr < rows_valid) {
        const uint8_t* p = base + (gr * s_r + (int64_t)gk * s_k) * EB;
        if (vec_ok && kcontig && gk + kCE <= K) {
          x = *(const i32x4*)p;
        } else {
          uint8_t bytes[16] = {};
#pragma unroll
          for (int e = 0; e < kCE; ++e) {
            if (gk + e < K) {
              const uint8_t* q = p + (int64_t)e * s_k * EB;
#pragma unroll
              for (int b = 0; b < EB; ++b) bytes[e * EB + b] = q[b];
            }
          }
          x = __builtin_bit_cast(i32x4, bytes);
        }
      }
      v[it] = x;
    }
  }

  __device__ __forceinline__ void store(uint8_t* slab, bool kcontig, int tid) const {
    constexpr StripMinedMap kmap(ROWS, kChunks, kThreads, 1, kI, 1);
    constexpr StripMinedMap rmap(ROWS, kChunks, kThreads, 1, kI, 0);
#pragma unroll
    for (int it = 0; it < kI; ++it) {
      const int r = kcontig ? kmap.row(tid, it, 0) : rmap.row(tid, it, 0);
      const int c = kcontig ? kmap.col(tid, it, 0) : rmap.col(tid, it, 0);
      *(i32x4*)(slab + r * kRowBytes + Swz::chunk(r, c) * 16) = v[it];
    }
  }
};

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
struct ConvSlab : RegSlab<ROWS, EB, kRowBytes> {
  using Base = RegSlab<ROWS, EB, kRowBytes>;

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

__device__ __forceinline__ float activate(float y, int act) {
  if (act == TLA_ACT_RELU) return y > 0.f ? y : 0.f;
  if (act == TLA_ACT_GELU) return 0.5f * y * (1.0f + erff(y * 0.70710678118654752f));
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
// The two fast epilogue paths below are compiled once per activation and
// per D type, so the per-element work is straight-line code; C and bias
// (bf16 or fp16) are widened with a select rather than a branch.
__device__ __forceinline__ float widen16(uint32_t w, bool bf16) {
  const float b = __builtin_bit_cast(float, w << 16);
  const float h = (float)__builtin_bit_cast(_Float16, (uint16_t)w);
  return bf16 ? b : h;
}

template <int kAct>
__device__ __forceinline__ float act_t(float y) {
  if constexpr (kAct == TLA_ACT_RELU) return y > 0.f ? y : 0.f;
  if constexpr (kAct == TLA_ACT_GELU) return 0.5f * y * (1.0f + erff(y * 0.70710678118654752f));
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

// y = act(alpha*acc + beta*c + bias) for the four values of group g of tile
// (i, j); c and bias arrive as packed 16-bit pairs.
template <int kAct, bool kDBf16>
__device__ __forceinline__ uint2 epi_group(const f32x16& acc, int g, uint2 c, uint2 b, float alpha,
                                           float beta, bool c_bf16, bool b_bf16) {
  const uint32_t cw[4] = {c.x, c.x >> 16, c.y, c.y >> 16};
  const uint32_t bw[4] = {b.x, b.x >> 16, b.y, b.y >> 16};
  float y[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v = alpha * acc[4 * g + q];
    v += beta * widen16(cw[q] & 0xFFFFu, c_bf16);
    y[q] = act_t<kAct>(v + widen16(bw[q] & 0xFFFFu, b_bf16));
  }
  return uint2{pack2<kDBf16>(y[0], y[1]), pack2<kDBf16>(y[2], y[3])};
}

// This lane's 16-bit bias values for its column groups, all loads issued
// before any is used (zero bits when there is no bias).
template <int FN>
__device__ __forceinline__ void load_bias16(const GemmParams& p, int n_base, int half,
                                            uint2 (&braw)[FN][4]) {
  static_for<FN>([&](auto j) { static_for<4>([&](auto g) { braw[j][g] = uint2{0u, 0u}; }); });
  if (p.bias) {
    const uint2* b = (const uint2*)((const uint16_t*)p.bias + n_base + 4 * half);
    static_for<FN>([&](auto j) { static_for<4>([&](auto g) { braw[j][g] = b[8 * j + 2 * g]; }); });
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
template <int kAct, bool kDBf16, int FM, int FN>
__device__ __forceinline__ void epilogue_lds(const GemmParams& p, int m_base, int n_base, int lane,
                                             const f32x16 (&acc)[FM][FN], uint8_t* region) {
  constexpr int kRowB = 64 * FN, kCh = kRowB / 16, kRowsPerKiB = 1024 / kRowB;
  static_assert(kCh == 4 || kCh == 8 || kCh == 16, "row width");
  constexpr int kIters = 32 * FM * kRowB / 1024;
  auto swz = [](int r, int c) { return c ^ ((r / (16 / kCh)) & (kCh - 1)); };
  const int row = lane & 31, half = lane >> 5;
  const int rr = lane / kCh, cs = lane % kCh;  // row-wise view of one KiB
  const bool has_c = p.beta != 0.f;
  if (has_c) {
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
  const bool c_bf16 = p.c_type == kBF16, b_bf16 = p.bias_type == kBF16;
  const float beta = has_c ? p.beta : 0.f;
  static_for<FM>([&](auto i) {
    static_for<FN>([&](auto j) {
      static_for<4>([&](auto g) {
        const int r = 32 * i + row;
        uint8_t* slot = region + r * kRowB + swz(r, 4 * j + g) * 16 + 8 * half;
        const uint2 c = has_c ? *(const uint2*)slot : uint2{0u, 0u};
        *(uint2*)slot = epi_group<kAct, kDBf16>(acc[i][j], g, c, braw[j][g], p.alpha, beta, c_bf16, b_bf16);
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

// Full wave tile straight from and to global memory with 8-byte vectors;
// all C and bias loads are issued before the arithmetic.
template <int kAct, bool kDBf16, int FM, int FN>
__device__ __forceinline__ void epilogue_direct(const GemmParams& p, int m_base, int n_base, int lane,
                                                const f32x16 (&acc)[FM][FN]) {
  const int row = lane & 31, half = lane >> 5;
  const bool has_c = p.beta != 0.f;
  uint2 c[FM][FN][4];
  if (has_c) {
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
  const bool c_bf16 = p.c_type == kBF16, b_bf16 = p.bias_type == kBF16;
  const float beta = has_c ? p.beta : 0.f;
  uint16_t* D = (uint16_t*)p.D;
  static_for<FM>([&](auto i) {
    static_for<FN>([&](auto j) {
      static_for<4>([&](auto g) {
        *(uint2*)(D + (int64_t)(m_base + 32 * i + row) * p.d_sm + n_base + 32 * j + 8 * g + 4 * half) =
            epi_group<kAct, kDBf16>(acc[i][j], g, c[i][j][g], braw[j][g], p.alpha, beta, c_bf16, b_bf16);
      });
    });
  });
}

template <bool kLds, int kAct, bool kDBf16, int FM, int FN>
__device__ __forceinline__ void epilogue_fast(const GemmParams& p, int m_base, int n_base, int lane,
                                              const f32x16 (&acc)[FM][FN], uint8_t* region) {
  if constexpr (kLds)
    epilogue_lds<kAct, kDBf16, FM, FN>(p, m_base, n_base, lane, acc, region);
  else
    epilogue_direct<kAct, kDBf16, FM, FN>(p, m_base, n_base, lane, acc);
}

template <bool kLds, int FM, int FN>
__device__ __forceinline__ void epilogue_switch(const GemmParams& p, int m_base, int n_base, int lane,
                                                const f32x16 (&acc)[FM][FN], uint8_t* region) {
  const bool dbf = p.d_type == kBF16;
  switch (p.act) {
    case TLA_ACT_RELU:
      if (dbf) epilogue_fast<kLds, TLA_ACT_RELU, true>(p, m_base, n_base, lane, acc, region);
      else epilogue_fast<kLds, TLA_ACT_RELU, false>(p, m_base, n_base, lane, acc, region);
      break;
    case TLA_ACT_GELU:
      if (dbf) epilogue_fast<kLds, TLA_ACT_GELU, true>(p, m_base, n_base, lane, acc, region);
      else epilogue_fast<kLds, TLA_ACT_GELU, false>(p, m_base, n_base, lane, acc, region);
      break;
    default:
      if (dbf) epilogue_fast<kLds, TLA_ACT_NONE, true>(p, m_base, n_base, lane, acc, region);
      else epilogue_fast<kLds, TLA_ACT_NONE, false>(p, m_base, n_base, lane, acc, region);
      break;
  }
}

// The epilogue of one wavefront's FM x FN grid of 32x32 accumulator tiles,
// rows m_base + 32i + lane%32, column groups n_base + 32j + 8g + 4(lane/32).
// `region` is this wave's 32*FM x 64*FN-byte piece of LDS, free for reuse
// (the caller has synchronised the workgroup after its last LDS read), or
// null.  A wave tile inside D with 16-bit C (or no C) and bias takes the LDS
// path when C and D rows allow 16-byte vectors, else the direct path with
// 8-byte vectors; anything else (edge tiles, fp32 C or bias, strided C or D)
// goes group by group through the predicated epilogue4.
template <int FM, int FN>
__device__ __forceinline__ void epilogue_tiles(const GemmParams& p, int m_base, int n_base, int lane,
                                               const f32x16 (&acc)[FM][FN], uint8_t* region) {
  const bool full = m_base + 32 * FM <= p.M && n_base + 32 * FN <= p.N;
  const bool b_ok = !p.bias || ((p.flags & kBiasVec) && p.bias_type != kF32);
  const bool c16 = p.c_type != kF32;
  if (full && b_ok && region && (p.flags & kD16) && (p.beta == 0.f || (c16 && (p.flags & kC16)))) {
    epilogue_switch<true, FM, FN>(p, m_base, n_base, lane, acc, region);
  } else if (full && b_ok && (p.flags & kDVec) && (p.beta == 0.f || (c16 && (p.flags & kCVec)))) {
    epilogue_switch<false, FM, FN>(p, m_base, n_base, lane, acc, region);
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

// Both operands K-contiguous with 16-byte aligned rows, K a multiple of the
// slab width.  LDS holds kStages A slabs, then kStages B slabs; k-tile kt
// lives in slot kt % kStages of both.
//
// Schedule (one software pipeline over every MFMA k-step of every tile):
//  * the direct global -> LDS copies of tile kt + kStages - 1 are issued one
//    instruction at a time between the MFMAs of tile kt, so copy issue never
//    blocks the matrix cores;
//  * the fragments of step g+1 are read from LDS at the start of step g;
//  * half-way through the last step of tile kt every wave waits for tile
//    kt+1 and meets at one barrier, which also frees tile kt-1's slot for
//    the next copy.
// Past the end of K the copies reload the last k-tile, so every tile issues
// the same number of copies and the wait counts are constants.
//
// Addressing is out of the loop: a copy is a buffer load with a per-lane
// offset fixed for the whole kernel plus the tile's K offset in a scalar
// register, and a fragment read is one of a few per-lane base registers
// plus an immediate (slot and tile row).  The XOR swizzle only sees row bits
// below 32, so one base per k-step serves every 32-row fragment; grouping
// the A slots and the B slots keeps every immediate below 64 KiB.
template <int kCode, int BM, int BN, int kRowBytes, int kStages, int kFront = 0, int kWM = 2,
          int kWN = 2, bool kConv = false>
__global__ __launch_bounds__(64 * kWM * kWN) void gemm_fast_kernel(const GemmParams p) {
  using Atom = MfmaAtom<kCode>;
  using Frag = typename Atom::Frag;
  using Swz = typename Slab<kRowBytes>::Swz;
  constexpr int NT = 64 * kWM * kWN;  // kWM x kWN wavefronts
  constexpr int EB = elem_bytes(kCode);
  constexpr int BK = kRowBytes / EB;
  constexpr int WM = BM / kWM, WN = BN / kWN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int KSTEPS = BK / Atom::kK;
  static_assert(BK % Atom::kK == 0 && KSTEPS >= 2 && KSTEPS % 2 == 0,
                "fragment buffers alternate per step");
  static_assert(kStages >= 2, "copies need a free slot");
  constexpr int SLAB_A = BM * kRowBytes, SLAB_B = BN * kRowBytes;
  constexpr int B_BASE = kStages * SLAB_A;
  static_assert(kStages * (SLAB_A + SLAB_B) <= 160 * 1024, "LDS budget");
  static_assert(kStages * SLAB_A <= 65536 && kStages * SLAB_B <= 65536, "fragment immediates");
  constexpr int kChunks = Slab<kRowBytes>::kChunks;
  static_assert((1 << Slab<kRowBytes>::kRowShift) * kChunks <= 32, "swizzle period divides 32 rows");
  constexpr int IA = BM * kChunks / NT, IB = BN * kChunks / NT;
  static_assert(IA * NT == BM * kChunks && IB * NT == BN * kChunks, "whole copy instructions");
  constexpr int kLoads = IA + IB;                  // copies per thread per tile
  constexpr int kSub = Atom::kLaneBytes / 16;      // 16-byte reads per fragment
  constexpr int kReads = (FM + FN) * kSub;
  constexpr int kMfmas = FM * FN;
  constexpr int kStepBytes = Atom::kK * EB;
  // Copies per full step, the rest go into the first half of the last step.
  // kFront > 0 puts all copies into the first kFront steps instead.
  constexpr int kSpread = kFront > 0 && kFront < KSTEPS ? kFront : KSTEPS;
  constexpr int kPerStep = (kLoads + kSpread - 1) / kSpread;
  constexpr int kFull = kPerStep * (KSTEPS - 1) < kLoads ? kPerStep * (KSTEPS - 1) : kLoads;
  constexpr int kLast = kLoads - kFull;
  constexpr int kWait = (kStages - 2) * kLoads;  // copies allowed in flight past the next tile
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * (SLAB_A + SLAB_B)];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  schedule(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm0 = (wave % kWM) * WM, wn0 = (wave / kWM) * WN;
  const int KT = p.K / BK;

  // Copy q (A for q < IA, else B): slab row r = tid/kChunks + (NT/kChunks)*q',
  // landing at slab slot wave*64 + NT*q' (lane-linear); the lane fetches the
  // global chunk the swizzle assigns to that slot, from row r clamped to the
  // matrix (rows past M or N are never stored).
  uint32_t off[kLoads];
  static_for<kLoads>([&](auto q) {
    constexpr bool kA = q < IA;
    constexpr int qq = kA ? q : q - IA;
    const int r = tid / kChunks + (NT / kChunks) * qq;
    const int64_t row = kA ? min(m0 + r, p.M - 1) : min(n0 + r, p.N - 1);
    const int64_t rb = (kA ? p.a_sr : p.b_sr) * EB;
    off[q] = (uint32_t)(row * rb + Swz::chunk(r, tid % kChunks) * 16);
  });
  // Implicit-GEMM convolution: A row m is the output pixel (n, p, q); a
  // k-tile is 128 bytes of channels of one filter tap (C is a multiple of
  // the tile), so the tap is uniform and each lane keeps its pixel's image
  // origin (h0, w0) and byte offset.  Rows past M get an origin that no
  // tap brings into the image.
  int ch0[kConv ? IA : 1], cw0[kConv ? IA : 1];
  if constexpr (kConv) {
    static_for<IA>([&](auto q) {
      const int r = tid / kChunks + (NT / kChunks) * q;
      const int m = m0 + r;
      const int PQ = p.cP * p.cQ;
      const int n = m / PQ, pq = m - n * PQ, pp = pq / p.cQ, qq = pq - pp * p.cQ;
      const int h0 = pp * p.cu - p.cph, w0 = qq * p.cv - p.cpw;
      const bool live = m < p.M;
      ch0[q] = live ? h0 : -0x40000000;
      cw0[q] = w0;
      const int64_t base = (((int64_t)n * p.cH + h0) * p.cW + w0) * p.cC * EB;
      off[q] = (uint32_t)(live ? base : 0) + Swz::chunk(r, tid % kChunks) * 16;
    });
  }
  const int x_records = kConv ? (int)((int64_t)p.M / (p.cP * p.cQ) * p.cH * p.cW * p.cC * EB) : 0;
  // Fragment bases for each k-step (and each 16-byte half of a 32-byte
  // fragment): row wm0 + lane%32 of the A slot, wn0 + lane%32 of the B slot.
  uint32_t fa[KSTEPS][kSub], fb[KSTEPS][kSub];
  static_for<KSTEPS>([&](auto ks) {
    static_for<kSub>([&](auto u) {
      const int c = (ks * kStepBytes + (lane >> 5) * Atom::kLaneBytes) / 16 + u;
      const int ra = wm0 + (lane & 31), rb = wn0 + (lane & 31);
      fa[ks][u] = (uint32_t)(ra * kRowBytes + Swz::chunk(ra, c) * 16);
      fb[ks][u] = (uint32_t)(B_BASE + rb * kRowBytes + Swz::chunk(rb, c) * 16);
    });
  });

  f32x16 acc[FM][FN];
  static_for<FM>([&](auto i) { static_for<FN>([&](auto j) { acc[i][j] = f32x16{}; }); });
  Frag a[2][FM], b[2][FN];
  auto lds_frag = [&](const uint32_t (&base)[kSub], int imm) -> Frag {
    if constexpr (kSub == 1) {
      return *(const i32x4*)(smem + base[0] + imm);
    } else {
      const i32x4 lo = *(const i32x4*)(smem + base[0] + imm);
      const i32x4 hi = *(const i32x4*)(smem + base[1] + imm);
      return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  auto read_frags = [&](auto buf, auto slot, auto ks) {
    static_for<FM>([&](auto i) { a[buf][i] = lds_frag(fa[ks], slot * SLAB_A + i * 32 * kRowBytes); });
    static_for<FN>([&](auto j) { b[buf][j] = lds_frag(fb[ks], slot * SLAB_B + j * 32 * kRowBytes); });
  };
  auto mma = [&](auto buf, auto idx) {
    Atom::mma(acc[idx / FN][idx % FN], b[buf][idx % FN], a[buf][idx / FN]);
  };
  // copy q of tile t into slot `slot`; tiles past K reload the last one
  auto copy = [&](int t, auto slot, auto q) {
    const uint32_t kb = (uint32_t)min(t, KT - 1) * kRowBytes;
    if constexpr (q < IA && kConv) {
      const int k0 = min(t, KT - 1) * BK;  // first channel of the tap, uniform
      const int rs = k0 / p.cC, c0 = k0 - rs * p.cC;
      const int fr = rs / p.cS, fs = rs - fr * p.cS;
      const int dh = fr * p.cdh, dw = fs * p.cdw;
      const int h = ch0[q] + dh, w = cw0[q] + dw;
      const bool in = (unsigned)h < (unsigned)p.cH && (unsigned)w < (unsigned)p.cW;
      // modulo 2^32, like off[q]: their sum is the tap's true offset (below
      // 2^31) whenever the tap is inside the image
      const uint32_t tap = (((uint32_t)dh * (uint32_t)p.cW + (uint32_t)dw) * (uint32_t)p.cC +
                            (uint32_t)c0) * (uint32_t)EB;
      dma16_buf(p.A, in ? off[q] + tap : 0xFFFFFFF0u, 0,
                smem + slot * SLAB_A + (wave * 64 + NT * q) * 16, x_records);
    } else if constexpr (q < IA)
      dma16_buf(p.A, off[q], kb, smem + slot * SLAB_A + (wave * 64 + NT * q) * 16);
    else
      dma16_buf(p.B, off[q], kb, smem + B_BASE + slot * SLAB_B + (wave * 64 + NT * (q - IA)) * 16);
  };
  // MFMAs [lo, hi) of a step with copies [q0, q0 + nq) of tile t spread
  // evenly between them: after MFMA k come copies [k*nq/n, (k+1)*nq/n).
  auto mfmas_with_copies = [&](auto buf, auto lo, auto hi, int t, auto slot, auto q0, auto nq) {
    constexpr int n = hi - lo;
    static_for<n>([&](auto k) {
      mma(buf, std::integral_constant<int, lo + k>{});
      constexpr int c0 = k * nq / n, c1 = (k + 1) * nq / n;
      static_for<c1 - c0>([&](auto c) { copy(t, slot, std::integral_constant<int, q0 + c0 + c>{}); });
    });
    static_for<n>([&](auto k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      constexpr int c0 = k * nq / n, c1 = (k + 1) * nq / n;
      if constexpr (c1 > c0) __builtin_amdgcn_sched_group_barrier(0x020, c1 - c0, 0);
    });
  };
  // k-tile kt, which lives in slot S (= kt % kStages)
  auto tile = [&](int kt, auto S) {
    using Next = std::integral_constant<int, (S + 1) % kStages>;
    using Fill = std::integral_constant<int, (S + kStages - 1) % kStages>;
    const int ct = kt + kStages - 1;  // tile whose copies are issued now
    static_for<KSTEPS>([&](auto ks) {
      constexpr int cur = ks & 1;
      if constexpr (ks + 1 < KSTEPS) {
        read_frags(std::integral_constant<int, cur ^ 1>{}, S, std::integral_constant<int, ks + 1>{});
        __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
        constexpr int q0 = ks * kPerStep < kFull ? ks * kPerStep : kFull;
        constexpr int q1 = (ks + 1) * kPerStep < kFull ? (ks + 1) * kPerStep : kFull;
        mfmas_with_copies(std::integral_constant<int, cur>{}, std::integral_constant<int, 0>{},
                          std::integral_constant<int, kMfmas>{}, ct, Fill{},
                          std::integral_constant<int, q0>{}, std::integral_constant<int, q1 - q0>{});
      } else {
        mfmas_with_copies(std::integral_constant<int, cur>{}, std::integral_constant<int, 0>{},
                          std::integral_constant<int, kMfmas / 2>{}, ct, Fill{},
                          std::integral_constant<int, kFull>{}, std::integral_constant<int, kLast>{});
        if (kt + 1 < KT) {
          wait_vmcnt<kWait>();  // tile kt+1 landed (this thread's copies)
          stage_barrier();      // ... everyone's; tile kt-1's slot is free
          read_frags(std::integral_constant<int, cur ^ 1>{}, Next{}, std::integral_constant<int, 0>{});
        }
        static_for<kMfmas - kMfmas / 2>([&](auto k) {
          mma(std::integral_constant<int, cur>{}, std::integral_constant<int, kMfmas / 2 + k>{});
        });
      }
    });
  };

  if (KT > 0) {
    static_for<kStages - 1>([&](auto t) {
      static_for<kLoads>([&](auto q) { copy(t, t, q); });
    });
    wait_vmcnt<kWait>();
    stage_barrier();
    read_frags(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{},
               std::integral_constant<int, 0>{});
    for (int kt = 0; kt < KT; kt += kStages) {
      static_for<kStages>([&](auto s) {
        if (kt + s < KT) tile(kt + s, s);
      });
    }
    wait_vmcnt<0>();  // no copy may land in LDS after this point
  }

  // Every wave is past its last LDS read: the slots become the waves'
  // epilogue regions.
  constexpr bool kLdsEpi = (NT / 64) * WM * 64 * FN <= kStages * (SLAB_A + SLAB_B);
  __syncthreads();
  epilogue_tiles<FM, FN>(p, m0 + wm0, n0 + wn0, lane, acc,
                         kLdsEpi ? smem + wave * WM * 64 * FN : nullptr);
}

// ------------------------------------------------------------------ kernel
// kStages LDS stages of BM + BN rows of kRowBytes bytes each.  K-tile kt
// lives in stage kt % kStages; up to kStages - 1 tiles are in flight, so the
// copy of a tile has kStages - 1 tiles of matrix-core work to arrive in.
template <int kCode, int BM, int BN, int kRowBytes, int kStages, bool kFast, bool kConv = false>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const GemmParams p) {
  using Atom = MfmaAtom<kCode>;
  using Frag = typename Atom::Frag;
  constexpr int EB = elem_bytes(kCode);
  constexpr int BK = kRowBytes / EB;         // K elements per k-tile
  constexpr int WM = BM / 2, WN = BN / 2;    // 2 x 2 wavefronts
  constexpr int FM = WM / 32, FN = WN / 32;  // MFMA tiles per wave
  constexpr int KSTEPS = BK / Atom::kK;
  static_assert(KSTEPS >= 1 && BK % Atom::kK == 0, "slab narrower than one MFMA step");
  constexpr int SLAB_A = BM * kRowBytes, STAGE = (BM + BN) * kRowBytes;
  static_assert(kStages * STAGE <= 160 * 1024, "LDS budget");
  // global_load_lds instructions one thread issues per k-tile
  constexpr int kLoadsPerTile = (BM + BN) * kRowBytes / 16 / kThreads;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tm, tn;
  schedule(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm0 = (wave & 1) * WM, wn0 = (wave >> 1) * WN;

  f32x16 acc[FM][FN];
  static_for<FM>([&](auto i) { static_for<FN>([&](auto j) { acc[i][j] = f32x16{}; }); });

  // Fragment double buffer and the pieces of one MFMA k-step.
  Frag a[2][FM], b[2][FN];
  auto read_frags = [&](auto buf, const uint8_t* stage, auto ks) {
    static_for<FM>([&](auto i) {
      a[buf][i] = load_frag<kCode, kRowBytes>(stage, wm0 + 32 * i + (lane & 31), ks, lane);
    });
    static_for<FN>([&](auto j) {
      b[buf][j] = load_frag<kCode, kRowBytes>(stage + SLAB_A, wn0 + 32 * j + (lane & 31), ks, lane);
    });
  };
  // MFMAs number lo .. hi-1 of a step (i major, j minor)
  auto mfmas = [&](auto buf, auto lo, auto hi) {
    static_for<hi - lo>([&](auto q) {
      constexpr int idx = lo + q;
      Atom::mma(acc[idx / FN][idx % FN], b[buf][idx % FN], a[buf][idx / FN]);
    });
  };
  constexpr int kReads = (FM + FN) * (Atom::kLaneBytes / 16);
  constexpr int kMfmas = FM * FN;

  const int KT = (p.K + BK - 1) / BK;
  if constexpr (kFast) {
    // One software pipeline over all k-steps.  The fragments of step g+1 are
    // read at the start of step g, a whole step of MFMAs before use.  In the
    // last step of k-tile kt, half-way through its MFMAs, every wave waits
    // for tile kt+1 and meets at a barrier; that barrier also proves every
    // wave is done reading tile kt's stage, which is refilled at once with
    // tile kt+kStages.
    static_assert(KSTEPS % 2 == 0, "fragment buffers alternate per step");
    const int64_t a_rb = p.a_sr * EB, b_rb = p.b_sr * EB;
    auto issue = [&](int kt) {
      uint8_t* st = smem + (kt % kStages) * STAGE;
      const int64_t kb = (int64_t)kt * kRowBytes;
      dma_slab<BM, kRowBytes>(p.A, a_rb, m0, p.M, kb, st, tid);
      dma_slab<BN, kRowBytes>(p.B, b_rb, n0, p.N, kb, st + SLAB_A, tid);
    };
    // wait until tile `t` has landed, given tiles up to `last_issued` were issued
    auto wait_tile = [&](int t, int last_issued) {
      const int after = min(kStages - 1, last_issued - t);
      static_for<kStages>([&](auto n) {
        if (after == n) wait_vmcnt<n * kLoadsPerTile>();
      });
    };
    static_for<kStages>([&](auto s) {
      if (s < KT) issue(s);
    });
    if (KT > 0) {
      wait_tile(0, min(kStages, KT) - 1);
      __syncthreads();
      read_frags(std::integral_constant<int, 0>{}, smem, std::integral_constant<int, 0>{});
    }
    for (int kt = 0; kt < KT; ++kt) {
      const uint8_t* stage = smem + (kt % kStages) * STAGE;
      static_for<KSTEPS>([&](auto ks) {
        constexpr int cur = ks & 1;
        if constexpr (ks + 1 < KSTEPS) {
          read_frags(std::integral_constant<int, cur ^ 1>{}, stage,
                     std::integral_constant<int, ks + 1>{});
          mfmas(std::integral_constant<int, cur>{}, std::integral_constant<int, 0>{},
                std::integral_constant<int, kMfmas>{});
          __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, kMfmas, 0);
        } else {
          mfmas(std::integral_constant<int, cur>{}, std::integral_constant<int, 0>{},
                std::integral_constant<int, kMfmas / 2>{});
          if (kt + 1 < KT) {
            // tiles issued so far: 0 .. min(kt + kStages - 1, KT - 1)
            wait_tile(kt + 1, min(kt + kStages - 1, KT - 1));
            __syncthreads();
            if (kt + kStages < KT) issue(kt + kStages);
            read_frags(std::integral_constant<int, cur ^ 1>{},
                       smem + ((kt + 1) % kStages) * STAGE, std::integral_constant<int, 0>{});
          }
          mfmas(std::integral_constant<int, cur>{}, std::integral_constant<int, kMfmas / 2>{},
                std::integral_constant<int, kMfmas>{});
        }
      });
    }
  } else {
    static_assert(kStages == 2, "register-staged path double-buffers");
    // k-steps of one tile from LDS, fragments of step ks+1 read during ks
    auto compute = [&](const uint8_t* stage) {
      read_frags(std::integral_constant<int, 0>{}, stage, std::integral_constant<int, 0>{});
      static_for<KSTEPS>([&](auto ks) {
        constexpr int cur = ks & 1;
        if constexpr (ks + 1 < KSTEPS)
          read_frags(std::integral_constant<int, cur ^ 1>{}, stage,
                     std::integral_constant<int, ks + 1>{});
        mfmas(std::integral_constant<int, cur>{}, std::integral_constant<int, 0>{},
              std::integral_constant<int, kMfmas>{});
      });
    };
    static_assert(!kConv || !kFast, "the convolution view uses the register-staged path");
    std::conditional_t<kConv, ConvSlab<BM, EB, kRowBytes>, RegSlab<BM, EB, kRowBytes>> ra;
    RegSlab<BN, EB, kRowBytes> rb;
    const bool a_vec = (p.flags >> 8) & 1, b_vec = (p.flags >> 9) & 1;
    const bool a_kc = (p.a_sk == 1), b_kc = (p.b_sk == 1);
    if (KT > 0) {
      if constexpr (kConv) ra.load_conv(p, m0, 0, a_vec, tid);
      else ra.load(p.A, p.a_sr, p.a_sk, m0, p.M, 0, p.K, a_vec, tid);
      rb.load(p.B, p.b_sr, p.b_sk, n0, p.N, 0, p.K, b_vec, tid);
      ra.store(smem, kConv || a_kc, tid);
      rb.store(smem + SLAB_A, b_kc, tid);
    }
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      uint8_t* cur = smem + (kt & 1) * STAGE;
      uint8_t* nxt = smem + ((kt + 1) & 1) * STAGE;
      if (kt + 1 < KT) {
        if constexpr (kConv) ra.load_conv(p, m0, (kt + 1) * BK, a_vec, tid);
        else ra.load(p.A, p.a_sr, p.a_sk, m0, p.M, (kt + 1) * BK, p.K, a_vec, tid);
        rb.load(p.B, p.b_sr, p.b_sk, n0, p.N, (kt + 1) * BK, p.K, b_vec, tid);
      }
      compute(cur);
      if (kt + 1 < KT) {
        ra.store(nxt, kConv || a_kc, tid);
        rb.store(nxt + SLAB_A, b_kc, tid);
      }
      __syncthreads();
    }
  }

  // Epilogue: acc[i][j] holds the D^T piece for rows m0+wm0+32i.. and
  // columns n0+wn0+32j..; value r of lane l sits at (row, col) =
  // (lane%32, mfma32_acc_row(l, r)) of that 32x32 piece.  No copy is in
  // flight here; after the barrier the stages are the waves' regions.
  constexpr bool kLdsEpi = 4 * WM * 64 * FN <= kStages * STAGE;
  __syncthreads();
  epilogue_tiles<FM, FN>(p, m0 + wm0, n0 + wn0, lane, acc,
                         kLdsEpi ? smem + wave * WM * 64 * FN : nullptr);
}

// ----------------------------------------------------------------- dispatch
bool aligned(const void* p, int64_t bytes) { return ((uintptr_t)p % (uintptr_t)bytes) == 0; }

void set_grid(GemmParams& p, int BM, int BN, int64_t* grid) {
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  *grid = (int64_t)p.tiles_m * p.tiles_n;
}

template <int kCode, int BM, int BN, int kRowBytes, int kStages, int kFront, int kWM, int kWN,
          bool kConv = false>
int launch_fast(const GemmParams& p0, hipStream_t stream) {
  GemmParams p = p0;
  int64_t grid;
  set_grid(p, BM, BN, &grid);
  if (grid <= 0) return TLA_OK;
  if (grid > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((gemm_fast_kernel<kCode, BM, BN, kRowBytes, kStages, kFront, kWM, kWN, kConv>),
                     dim3((unsigned)grid), dim3(64 * kWM * kWN), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
}

template <int kCode, int BM, int BN, int kRowBytes, bool kFast>
int launch_two_stage(const GemmParams& p0, hipStream_t stream) {
  GemmParams p = p0;
  int64_t grid;
  set_grid(p, BM, BN, &grid);
  if (grid <= 0) return TLA_OK;
  if (grid > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((gemm_kernel<kCode, BM, BN, kRowBytes, 2, kFast>), dim3((unsigned)grid),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
}

// The variants the library ships.  Every fast variant moves whole 128-byte
// K rows per copy (the direct-to-LDS copy rate per compute unit halves with
// every halving of the row width), so K must be a multiple of 128 bytes.
//   16-bit, >= 128 tiles of 256x256: 8 wavefronts (2x4, 128x64 each), two
//     stages, each tile's copies issued during the first MFMA step of the
//     tile before (measured ~1 % ahead of spreading them over two or all
//     four steps).
//   16-bit, smaller: 128x128, 4 wavefronts, three stages.
//   e4m3: the two-stage kernel (its 32-byte fragments do not fit the
//     8-wavefront register budget).
int fast_slab_bytes(int) { return 128; }

const char* const kVariantNames[kGemmVariants] = {"gemm_fast_256x256", "gemm_fast_128x128",
                                                  "gemm_general_128x128"};
const int kVariantTile[kGemmVariants] = {256, 128, 128};

template <int kCode>
int dispatch_typed(const GemmParams& p, bool fast, bool big, hipStream_t s, bool dry,
                   const char** name, int forced) {
  // e4m3: the 128x128 kernel (two workgroups per compute unit) measured
  // ahead of 256x256 at every size of the variant sweep (8192^3: 644 vs
  // 725 us), so it is the automatic choice whenever the fast layout holds.
  const bool use_big = big && kCode != kE4M3;
  const int v = forced >= 0 ? forced : (fast ? (use_big ? 0 : 1) : 2);
  if (v < 2 && !fast) return TLA_ERR_UNSUPPORTED;  // a fast variant needs the fast layout
  if (name) *name = kVariantNames[v];
  if (dry) return TLA_OK;
  if constexpr (kCode == kE4M3) {
    if (v == 0) return launch_two_stage<kCode, 256, 256, 128, true>(p, s);
    if (v == 1) return launch_two_stage<kCode, 128, 128, 128, true>(p, s);
  } else {
    if (v == 0) return launch_fast<kCode, 256, 256, 128, 2, 1, 2, 4>(p, s);
    // 8 wavefronts of 64 x 32 (two per SIMD): 9.2 us at 1024^3 and 20.3 us
    // at 2048^3, against 11.1 and 21.7 us for 4 wavefronts of 64 x 64
    if (v == 1) return launch_fast<kCode, 128, 128, 128, 3, 1, 2, 4>(p, s);
  }
  return launch_two_stage<kCode, 128, 128, 128, false>(p, s);
}

// The kernel each variant launches for operand type kCode.
template <int kCode>
const void* variant_kernel(int v, int* threads) {
  *threads = kThreads;
  if constexpr (kCode == kE4M3) {
    if (v == 0) return (const void*)gemm_kernel<kCode, 256, 256, 128, 2, true>;
    if (v == 1) return (const void*)gemm_kernel<kCode, 128, 128, 128, 2, true>;
  } else {
    if (v == 0) {
      *threads = 512;
      return (const void*)gemm_fast_kernel<kCode, 256, 256, 128, 2, 1, 2, 4>;
    }
    if (v == 1) {
      *threads = 512;
      return (const void*)gemm_fast_kernel<kCode, 128, 128, 128, 3, 1, 2, 4>;
    }
  }
  return (const void*)gemm_kernel<kCode, 128, 128, 128, 2, false>;
}

}  // namespace

int conv_dispatch(const ConvProblem& c, hipStream_t stream) {
  const int eb = elem_bytes(c.type);
  GemmParams p{};
  p.A = (const uint8_t*)c.x;
  p.B = (const uint8_t*)c.w;
  p.C = (const uint8_t*)c.C;
  p.D = (uint8_t*)c.y;
  p.bias = (const uint8_t*)c.bias;
  p.M = (int)(c.N * c.P * c.Q);
  p.N = (int)c.K;
  p.K = (int)(c.R * c.S * c.C_in);
  // B = the filter as K rows of R*S*C (K-contiguous); C and D are N*P*Q x K
  p.b_sr = p.K;
  p.b_sk = 1;
  p.c_sm = p.d_sm = c.K;
  p.c_sn = p.d_sn = 1;
  p.c_type = p.d_type = c.type;
  p.bias_type = c.bias_type;
  p.act = c.act;
  p.alpha = c.alpha;
  p.beta = c.C ? c.beta : 0.f;
  p.cH = (int)c.H; p.cW = (int)c.W; p.cC = (int)c.C_in; p.cR = (int)c.R; p.cS = (int)c.S;
  p.cP = (int)c.P; p.cQ = (int)c.Q; p.cu = c.u; p.cv = c.v; p.cph = c.ph; p.cpw = c.pw;
  p.cdh = c.dh; p.cdw = c.dw;
  if (c.C && (c.K % 4) == 0 && aligned(c.C, 8)) p.flags |= kCVec;
  if ((c.K % 4) == 0 && aligned(c.y, 8)) p.flags |= kDVec;
  if (c.C && (c.K % 8) == 0 && aligned(c.C, 16)) p.flags |= kC16;
  if ((c.K % 8) == 0 && aligned(c.y, 16)) p.flags |= kD16;
  if (c.bias && aligned(c.bias, 4 * elem_bytes(c.bias_type))) p.flags |= kBiasVec;
  const bool x_vec = (c.C_in * eb) % 16 == 0 && aligned(c.x, 16);
  const bool w_vec = ((int64_t)p.K * eb) % 16 == 0 && aligned(c.w, 16);
  p.flags |= (x_vec ? 1 << 8 : 0) | (w_vec ? 1 << 9 : 0);
  // Direct-to-LDS implicit GEMM when every 128-byte k-tile is channels of
  // one tap (C a multiple of 64), 16-byte aligned image and filter rows and
  // both operands below 2 GiB; otherwise the register-staged loader.
  const int64_t x_bytes = c.N * c.H * c.W * c.C_in * eb;
  const bool fast = (c.C_in * eb) % 128 == 0 && aligned(c.x, 16) && w_vec &&
                    x_bytes < (int64_t(1) << 31) && (int64_t)p.K * p.N * eb < (int64_t(1) << 31);
  // Tiles: with at most 64 output channels a 256 x 64 tile (a 128-wide one
  // would be half empty), else 128 x 128; two LDS stages either way, so two
  // workgroups share a CU and one's epilogue overlaps the other's main loop.
  // On 32 x 56 x 56 x 64 -> 64 (3x3) the 256 x 64 tile measured 19.5 us
  // against 40.5 us for three-stage 128 x 128 tiles; on 32 x 28 x 28 x 256
  // -> 256 two stages measured 45.4 us against 52.8 us for three.
  if (fast) {
    const bool narrow = c.K <= 64;
    if (c.type == TLA_BF16)
      return narrow ? launch_fast<kBF16, 256, 64, 128, 2, 1, 2, 2, true>(p, stream)
                    : launch_fast<kBF16, 128, 128, 128, 2, 1, 2, 2, true>(p, stream);
    return narrow ? launch_fast<kF16, 256, 64, 128, 2, 1, 2, 2, true>(p, stream)
                  : launch_fast<kF16, 128, 128, 128, 2, 1, 2, 2, true>(p, stream);
  }
  int64_t grid;
  set_grid(p, 128, 128, &grid);
  if (grid <= 0) return TLA_OK;
  if (grid > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
  if (c.type == TLA_BF16)
    hipLaunchKernelGGL((gemm_kernel<kBF16, 128, 128, 128, 2, false, true>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<kF16, 128, 128, 128, 2, false, true>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
}

int gemm_variant_info(int a_type, int variant, GemmKernelInfo* out) {
  if (variant < 0 || variant >= kGemmVariants) return TLA_ERR_INVALID_ARG;
  int threads = 0;
  const void* k = nullptr;
  switch (a_type) {
    case TLA_BF16: k = variant_kernel<kBF16>(variant, &threads); break;
    case TLA_F16: k = variant_kernel<kF16>(variant, &threads); break;
    case TLA_E4M3: k = variant_kernel<kE4M3>(variant, &threads); break;
    default: return TLA_ERR_UNSUPPORTED;
  }
  hipFuncAttributes attr{};
  if (hipFuncGetAttributes(&attr, k) != hipSuccess) return TLA_ERR_HIP;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k, threads, 0) != hipSuccess)
    return TLA_ERR_HIP;
  out->name = kVariantNames[variant];
  out->tile = kVariantTile[variant];
  out->threads = threads;
  out->lds_bytes = (int)attr.sharedSizeBytes;
  out->vgprs = attr.numRegs;
  out->blocks_per_cu = blocks;
  return TLA_OK;
}

int gemm_dispatch(const GemmProblem& g, hipStream_t stream, bool dry_run, const char** name,
                  int forced) {
  if (g.M > 0x7FFFFFFF || g.N > 0x7FFFFFFF || g.K > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
  const int eb = elem_bytes(g.a_type);
  GemmParams p{};
  p.A = (const uint8_t*)g.A;
  p.B = (const uint8_t*)g.B;
  p.C = (const uint8_t*)g.C;
  p.D = (uint8_t*)g.D;
  p.bias = (const uint8_t*)g.bias;
  // operand views as (row, k) layouts: A rows are m, B rows are n
  p.a_sr = g.a_order == TLA_ROW_MAJOR ? g.lda : 1;
  p.a_sk = g.a_order == TLA_ROW_MAJOR ? 1 : g.lda;
  p.b_sr = g.b_order == TLA_COL_MAJOR ? g.ldb : 1;
  p.b_sk = g.b_order == TLA_COL_MAJOR ? 1 : g.ldb;
  p.c_sm = g.c_order == TLA_ROW_MAJOR ? g.ldc : 1;
  p.c_sn = g.c_order == TLA_ROW_MAJOR ? 1 : g.ldc;
  p.d_sm = g.d_order == TLA_ROW_MAJOR ? g.ldd : 1;
  p.d_sn = g.d_order == TLA_ROW_MAJOR ? 1 : g.ldd;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  p.c_type = g.c_type;
  p.d_type = g.d_type;
  p.bias_type = g.bias_type;
  p.act = g.act;
  p.alpha = g.alpha_eff;
  p.beta = g.beta;
  if (!g.C) p.beta = 0.f;
  const int ceb = elem_bytes(g.c_type), beb = elem_bytes(g.bias_type);
  if (g.C && g.c_order == TLA_ROW_MAJOR && (g.ldc % 4) == 0 && aligned(g.C, 4 * ceb)) p.flags |= kCVec;
  if (g.d_order == TLA_ROW_MAJOR && (g.ldd % 4) == 0 && aligned(g.D, 8)) p.flags |= kDVec;
  if (g.C && ceb == 2 && g.c_order == TLA_ROW_MAJOR && (g.ldc % 8) == 0 && aligned(g.C, 16)) p.flags |= kC16;
  if (g.d_order == TLA_ROW_MAJOR && (g.ldd % 8) == 0 && aligned(g.D, 16)) p.flags |= kD16;
  if (g.bias && aligned(g.bias, 4 * beb)) p.flags |= kBiasVec;
  const bool a_vec = (g.a_order == TLA_ROW_MAJOR) && ((g.lda * eb) % 16 == 0) && aligned(g.A, 16);
  const bool b_vec = (g.b_order == TLA_COL_MAJOR) && ((g.ldb * eb) % 16 == 0) && aligned(g.B, 16);
  p.flags |= (a_vec ? 1 << 8 : 0) | (b_vec ? 1 << 9 : 0);
  const int BK = fast_slab_bytes(g.a_type) / eb;
  // the fast kernel addresses each operand with 32-bit offsets below 2^31
  const bool small_ops = (int64_t)g.M * g.lda * eb < (int64_t(1) << 31) &&
                         (int64_t)g.N * g.ldb * eb < (int64_t(1) << 31);
  const bool fast = a_vec && b_vec && small_ops && g.K > 0 && (g.K % BK) == 0;
  const int64_t tiles256 = ((g.M + 255) / 256) * ((g.N + 255) / 256);
  const bool big = tiles256 >= 128;
  switch (g.a_type) {
    case TLA_BF16: return dispatch_typed<kBF16>(p, fast, big, stream, dry_run, name, forced);
    case TLA_F16: return dispatch_typed<kF16>(p, fast, big, stream, dry_run, name, forced);
    case TLA_E4M3: return dispatch_typed<kE4M3>(p, fast, big, stream, dry_run, name, forced);
    default: return TLA_ERR_UNSUPPORTED;
  }
}

}  // namespace tla
