// gemm.hip -- the single-group direct-to-LDS GEMM kernels (128 x 128 and
// 256 x 256 block tiles), the implicit-GEMM convolution and the variant
// dispatch, for gfx950.
//
//   D = act(alpha_eff * A.B + beta*C + bias),  fp32 accumulation.
//
// Three levels of tiling, as in "CUTLASS / CuTe 主线" (hpc.payai.win/cutlass),
// section 一: a workgroup owns a BM x BN tile of D (the block tile), each of
// its 64-lane wavefronts a piece of it (the wave tile: 2 x 4 waves of
// (BM/2) x (BN/4) in gemm_fast_kernel with 16-bit operands, 2 x 2 waves of
// (BM/2) x (BN/2) in gemm_general.hip's kernel, which serves e4m3, the
// register-staged general path and the convolution), and each 32x32 MFMA
// instruction a
// 32x32 piece of that (the instruction tile).  The K loop (section 二's
// mainloop: global -> shared -> register) moves one 128-byte-wide K slab of
// A and of B per step into LDS (64 bf16/fp16 or 128 e4m3 per row), with two
// or three stages so the next slab streams in while the current one feeds
// the matrix cores (section 四: pipeline stages hide global latency).  The
// epilogue (gemm_common.hpp) applies alpha, beta*C, bias and the activation
// to the fp32 accumulators in registers and stores D once (section 四: fuse
// before the store).  The two-group 256 x 256 kernel the dispatch prefers
// for large problems lives in gemm_pingpong.hip.
//
// Load paths:
//   fast    both operands K-contiguous, 16-byte aligned rows, K a multiple of
//           the slab width: each lane issues a direct HBM -> LDS copy that
//           lands lane-linearly; the LDS XOR swizzle is applied by permuting
//           which global chunk each lane fetches.  Rows past M or N are
//           clamped to the last real row (their results are never stored),
//           so the loop carries no predicates.
//   general any order, pitch or alignment, ragged K (gemm_general.hip):
//           registers staged through a strip-mined thread map with
//           per-element predicates; elements outside the matrix load as
//           zero.
#include "gemm_common.hpp"

namespace tla {
namespace {

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
//
// kBT: B is N-contiguous (a row-major K x N matrix, 16-bit).  Its slab is
// BK rows of k, each BN columns of n (2*BN bytes, 16-byte chunk c of row r
// stored at chunk c ^ 4 (r % 4)), filled by the same direct copies; a B
// fragment (32 columns n x 16 k, lane l: column l % 32, k 8 (l / 32) .. + 7)
// is two ds_read_b64_tr_b16, each giving a lane four consecutive k of its
// column.  In a quarter-wave the instruction hands lane j element e from
// the 8 bytes addressed by lane 4 e + j / 4, at position j % 4; so lane a
// of the quarter-wave addresses row k0 + a / 4, columns n0 + 4 (a % 4) ..
// + 3, and lane j receives B[k0 .. k0 + 3][n0 + j].  The swizzle keeps the
// 32 lanes of one half-wave (rows k0 .. k0 + 3, 32 bytes each of two
// column groups) on 16 distinct 16-byte bank groups.
//
// kAT: A is M-contiguous (a column-major M x K matrix, 16-bit, M a multiple
// of 8), held the same way: BK rows of k, each BM columns of m, an A
// fragment two transpose reads per 32 rows of m (an A fragment has a B
// fragment's layout).  Rows of k past K lie past the copy's record count.
template <int kCode, int BM, int BN, int kRowBytes, int kStages, int kFront = 0, int kWM = 2,
          int kWN = 2, bool kConv = false, bool kBT = false, bool kAT = false>
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
  static_assert(!kBT || (EB == 2 && BN >= 128 && !kConv && kWN * 32 == BN),
                "N-contiguous B: 16-bit, one 32-column fragment per wave");
  static_assert(!kAT || (EB == 2 && BM >= 128 && !kConv), "M-contiguous A: 16-bit");
  constexpr int kRowBT = BN * 2;                   // bytes per k row of an N-contiguous slab
  constexpr int kChBT = kRowBT / 16;
  constexpr int kRowAT = BM * 2;                   // bytes per k row of an M-contiguous slab
  constexpr int kChAT = kRowAT / 16;
  static_assert(kStages * SLAB_A <= 65536 && kStages * SLAB_B <= 65536, "fragment immediates");
  constexpr int kChunks = Slab<kRowBytes>::kChunks;
  static_assert((1 << Slab<kRowBytes>::kRowShift) * kChunks <= 32, "swizzle period divides 32 rows");
  constexpr int IA = BM * kChunks / NT, IB = BN * kChunks / NT;
  static_assert(IA * NT == BM * kChunks && IB * NT == BN * kChunks, "whole copy instructions");
  constexpr int kLoads = IA + IB;                  // copies per thread per tile
  constexpr int kSub = Atom::kLaneBytes / 16;      // 16-byte reads per fragment
  constexpr int kReads = (kAT ? 2 * FM : FM * kSub) + (kBT ? 2 : FN * kSub);
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
  const int KT = (p.K + BK - 1) / BK;
  const int KTf = p.K / BK;  // whole k-tiles; tile KTf, if K ends inside it, is ragged

  // Copy q (A for q < IA, else B): slab row r = tid/kChunks + (NT/kChunks)*q',
  // landing at slab slot wave*64 + NT*q' (lane-linear); the lane fetches the
  // global chunk the swizzle assigns to that slot, from row r clamped to the
  // matrix (rows past M or N are never stored).
  uint32_t off[kLoads];
  static_for<kLoads>([&](auto q) {
    constexpr bool kA = q < IA;
    constexpr int qq = kA ? q : q - IA;
    if constexpr (kA && kAT) {
      // as for an N-contiguous B: k row r, stored chunk pc holding columns
      // m0 + 8 (pc ^ 4 (r % 4)) .. + 7, clamped to the last chunk of M
      const int sc = tid + NT * qq, r = sc / kChAT, pc = sc % kChAT;
      const int m = min(m0 + 8 * (pc ^ (4 * (r & 3))), p.M - 8);
      off[q] = (uint32_t)(((int64_t)r * p.a_sk + m) * EB);
    } else if constexpr (!kA && kBT) {
      // slab chunk tid + NT q': k row r, stored chunk pc, which holds logical
      // chunk pc ^ 4 (r % 4): columns n0 + 8 lc .. + 7, clamped to the last
      // whole chunk of the matrix (columns past N are never stored)
      const int sc = tid + NT * qq, r = sc / kChBT, pc = sc % kChBT;
      const int n = min(n0 + 8 * (pc ^ (4 * (r & 3))), p.N - 8);
      off[q] = (uint32_t)(((int64_t)r * p.b_sk + n) * EB);
    } else {
      const int r = tid / kChunks + (NT / kChunks) * qq;
      const int64_t row = kA ? min(m0 + r, p.M - 1) : min(n0 + r, p.N - 1);
      const int64_t rb = (kA ? p.a_sr : p.b_sr) * EB;
      off[q] = (uint32_t)(row * rb + Swz::chunk(r, tid % kChunks) * 16);
    }
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
  // The ragged last k-tile (K a multiple of the 16-byte chunk): bit q is set
  // when copy q's K-contiguous chunk lies past K -- that copy then reads from
  // past every record and the range check returns zeros.  An N-contiguous B
  // slab's rows past K lie past its record count (K rows).
  uint32_t tail_past = 0;
  if constexpr (!kConv) {
    static_for<kLoads>([&](auto q) {
      constexpr bool kA = q < IA;
      constexpr int qq = kA ? q : q - IA;
      if constexpr (kA ? !kAT : !kBT) {
        const int r = tid / kChunks + (NT / kChunks) * qq;
        if (Swz::chunk(r, tid % kChunks) * 16 >= (p.K - KTf * BK) * EB) tail_past |= 1u << q;
      }
    });
  }
  const int b_records = kBT ? (int)min((int64_t)p.K * p.b_sk * EB, (int64_t)0x7FFFFFFF) : 0;
  const int a_records = kAT ? (int)min((int64_t)p.K * p.a_sk * EB, (int64_t)0x7FFFFFFF) : 0;
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
  // N-contiguous B: the two transpose reads of k-step ks (k0 = 16 ks +
  // 8 (quarter-wave / 2) + 4 h) for lane a = lane % 16 of its quarter-wave
  uint32_t fbt[kBT ? KSTEPS : 1][2];
  if constexpr (kBT) {
    const int qw = lane >> 4, a4 = lane & 15;
    static_for<KSTEPS>([&](auto ks) {
      static_for<2>([&](auto h) {
        const int k = 16 * ks + 8 * (qw >> 1) + 4 * h + (a4 >> 2);
        const int n = wn0 + 16 * (qw & 1) + 4 * (a4 & 3);
        fbt[ks][h] = (uint32_t)(B_BASE + k * kRowBT + (((n >> 3) ^ (4 * (k & 3))) * 16) +
                                (n & 7) * 2);
      });
    });
  }

  // M-contiguous A: the same two reads for each 32-row fragment i (the
  // swizzle does not commute with the 32-row step, so each has its bases)
  uint32_t fat[kAT ? KSTEPS : 1][kAT ? FM : 1][2];
  if constexpr (kAT) {
    const int qw = lane >> 4, a4 = lane & 15;
    static_for<KSTEPS>([&](auto ks) {
      static_for<FM>([&](auto i) {
        static_for<2>([&](auto h) {
          const int k = 16 * ks + 8 * (qw >> 1) + 4 * h + (a4 >> 2);
          const int m = wm0 + 32 * i + 16 * (qw & 1) + 4 * (a4 & 3);
          fat[ks][i][h] = (uint32_t)(k * kRowAT + (((m >> 3) ^ (4 * (k & 3))) * 16) + (m & 7) * 2);
        });
      });
    });
  }

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
  auto lds_frag_t = [&](const uint32_t (&base)[2], int imm) -> Frag {
    typedef int s32x2 __attribute__((ext_vector_type(2)));
    const s16x4 lo = ds_read_tr16(smem + base[0] + imm);
    const s16x4 hi = ds_read_tr16(smem + base[1] + imm);
    const s32x2 l2 = __builtin_bit_cast(s32x2, lo), h2 = __builtin_bit_cast(s32x2, hi);
    return Frag{l2[0], l2[1], h2[0], h2[1]};
  };
  auto read_frags = [&](auto buf, auto slot, auto ks) {
    if constexpr (kAT)
      static_for<FM>([&](auto i) { a[buf][i] = lds_frag_t(fat[ks][i], slot * SLAB_A); });
    else
      static_for<FM>([&](auto i) { a[buf][i] = lds_frag(fa[ks], slot * SLAB_A + i * 32 * kRowBytes); });
    if constexpr (kBT)
      b[buf][0] = lds_frag_t(fbt[ks], slot * SLAB_B);
    else
      static_for<FN>([&](auto j) { b[buf][j] = lds_frag(fb[ks], slot * SLAB_B + j * 32 * kRowBytes); });
  };
  auto mma = [&](auto buf, auto idx) {
    Atom::mma(acc[idx / FN][idx % FN], b[buf][idx % FN], a[buf][idx / FN]);
  };
  // copy q of tile t into slot `slot`; tiles past K reload the last one
  auto copy = [&](int t, auto slot, auto q) {
    const int tt = min(t, KT - 1);
    const uint32_t kb = (uint32_t)tt * kRowBytes;
    const uint32_t o = (tt == KTf && ((tail_past >> q) & 1)) ? 0x80000000u : off[q];
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
    } else if constexpr (q < IA && kAT)
      dma16_buf(p.A, off[q], (uint32_t)(tt * BK) * (uint32_t)(p.a_sk * EB),
                smem + slot * SLAB_A + (wave * 64 + NT * q) * 16, a_records);
    else if constexpr (q < IA)
      dma16_buf(p.A, o, kb, smem + slot * SLAB_A + (wave * 64 + NT * q) * 16);
    else if constexpr (kBT)
      dma16_buf(p.B, off[q], (uint32_t)(tt * BK) * (uint32_t)(p.b_sk * EB),
                smem + B_BASE + slot * SLAB_B + (wave * 64 + NT * (q - IA)) * 16, b_records);
    else
      dma16_buf(p.B, o, kb, smem + B_BASE + slot * SLAB_B + (wave * 64 + NT * (q - IA)) * 16);
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

// ----------------------------------------------------------------- dispatch
template <int kCode, int BM, int BN, int kRowBytes, int kStages, int kFront, int kWM, int kWN,
          bool kConv = false, bool kBT = false, bool kAT = false>
int launch_fast(const GemmParams& p0, hipStream_t stream) {
  GemmParams p = p0;
  int64_t grid;
  set_grid(p, BM, BN, &grid);
  if (grid <= 0) return TLA_OK;
  if (grid > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((gemm_fast_kernel<kCode, BM, BN, kRowBytes, kStages, kFront, kWM, kWN, kConv,
                                       kBT, kAT>),
                     dim3((unsigned)grid), dim3(64 * kWM * kWN), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
}

// The variants the library ships.  Every fast variant moves whole 128-byte
// K rows per copy (the direct-to-LDS copy rate per compute unit halves with
// every halving of the row width).  K need only be a multiple of the 16-byte
// chunk: the last k-tile's chunks past K read zeros through the buffer range
// check -- except in e4m3's 128 x 128 and 256 x 256 kernels, which copy
// through global_load_lds and need whole 128-byte rows.
//   0 two-group 256x256 kernel (gemm_pingpong.hip), any operand type: two
//     groups of four wavefronts (2x2 waves of 64x128 each) alternate
//     between MFMA-only and memory phases.
//   1 128x128 tiles.  16-bit: 8 wavefronts (2x4 of 64x32), three stages;
//     e4m3: the 4-wavefront (2x2 of 64x64) two-stage kernel.
//   2 the register-staged general kernel, 128x128, 4 wavefronts (2x2).
//   3 the single-group 256x256 kernel.  16-bit: 8 wavefronts (2x4 of
//     128x64), two stages, each tile's copies issued between the MFMAs of
//     the first k-step of the tile before; e4m3: 4 wavefronts (2x2 of
//     128x128), two stages.
int fast_slab_bytes(int) { return 128; }

const char* const kVariantNames[kGemmVariants] = {"gemm_pingpong_256x256", "gemm_fast_128x128",
                                                  "gemm_general_128x128", "gemm_fast_256x256"};
const int kVariantTile[kGemmVariants] = {256, 128, 128, 256};

// `bt`: not the fast layout, but A is and B is N-contiguous (16-bit, whole
// 16-byte chunks of n): variant 1's kernel takes B through LDS transpose
// reads.
template <int kCode>
int dispatch_typed(const GemmParams& p, bool fast, bool bt, bool at, bool big, bool k_slab,
                   hipStream_t s, bool dry, const char** name, int forced) {
  // N-contiguous B: the two-group kernel's transpose-read form from 128 tiles
  // of 256 x 256 on, as in the fast layout, the 128 x 128 kernel below (bf16,
  // four alternating rounds, medians: 4096^3 with C, bias and ReLU 109.4
  // against 139.3 us, 8192^2 x 2048 213.7 against 283.5 us, 3072^2 x 4096,
  // 144 tiles, 79.9 against 91.9 us; 2048^3 38.8 against 20.1 us)
  // M-contiguous 16-bit A (`at`): the same rule
  int v = forced >= 0 ? forced : ((fast || bt || at) ? (big ? 0 : 1) : 2);
  // a fast variant needs the fast layout (variants 0 and 1 also take `bt`
  // and `at`)
  if (v != 2 && !fast && !(v <= 1 && (bt || at))) return TLA_ERR_UNSUPPORTED;
  // e4m3's 128 x 128 and 256 x 256 kernels copy whole 128-byte slabs with no
  // range check: K off the slab takes the two-group kernel or the general one
  if constexpr (kCode == kE4M3) {
    if (!k_slab && v == 1 && forced < 0) v = 2;
    if (!k_slab && (v == 1 || v == 3)) return TLA_ERR_UNSUPPORTED;
  }
  if (name) *name = kVariantNames[v];
  if (dry) return TLA_OK;
  if constexpr (kCode != kE4M3) {
    if (v == 0 && at) return launch_pingpong(p, kCode, s, p.b_sk != 1, true);
    if (v == 1 && at) {
      if (p.b_sk != 1) return launch_fast<kCode, 128, 128, 128, 3, 1, 2, 4, false, true, true>(p, s);
      return launch_fast<kCode, 128, 128, 128, 3, 1, 2, 4, false, false, true>(p, s);
    }
    if (v == 0 && !fast) return launch_pingpong(p, kCode, s, true);
    if (v == 1 && !fast) return launch_fast<kCode, 128, 128, 128, 3, 1, 2, 4, false, true>(p, s);
  }
  if (v == 0) return launch_pingpong(p, kCode, s);
  if constexpr (kCode == kE4M3) {
    if (v == 3) return launch_two_stage_e4m3(p, true, s);
    if (v == 1) return launch_two_stage_e4m3(p, false, s);
  } else {
    if (v == 3) return launch_fast<kCode, 256, 256, 128, 2, 1, 2, 4>(p, s);
    // 8 wavefronts of 64 x 32 (two per SIMD): 9.2 us at 1024^3 and 20.3 us
    // at 2048^3, against 11.1 and 21.7 us for 4 wavefronts of 64 x 64
    if (v == 1) return launch_fast<kCode, 128, 128, 128, 3, 1, 2, 4>(p, s);
  }
  return launch_general(p, kCode, s);
}

// The kernel each variant launches for operand type kCode.
template <int kCode>
const void* variant_kernel(int v, int* threads) {
  *threads = kThreads;
  if (v == 0) {
    *threads = 512;
    return pingpong_kernel(kCode);
  }
  if constexpr (kCode == kE4M3) {
    if (v == 3) return two_stage_e4m3_kernel(true);
    if (v == 1) return two_stage_e4m3_kernel(false);
  } else {
    if (v == 3) {
      *threads = 512;
      return (const void*)gemm_fast_kernel<kCode, 256, 256, 128, 2, 1, 2, 4>;
    }
    if (v == 1) {
      *threads = 512;
      return (const void*)gemm_fast_kernel<kCode, 128, 128, 128, 3, 1, 2, 4>;
    }
  }
  return general_kernel(kCode);
}

}  // namespace

// The slab convolution of conv_slab.hip for 64 input and 64 output channels
// at stride 1 (image and filter 16-byte aligned, H*W*128 below 2^31); p is
// the implicit-GEMM view built below.  TLA_ERR_UNSUPPORTED when no slab of
// whole output rows fits LDS beside the filter.
int launch_conv_slab(const GemmParams& p, int type, hipStream_t stream);

int conv_dispatch(const ConvProblem& c, hipStream_t stream, int forced) {
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
  // 64 -> 64 channels at stride 1: the image slab and the whole filter in
  // LDS, each image element copied in once instead of once per tap (on
  // 32 x 56 x 56 x 64 -> 64, 3x3: 14.7 us against 17.8 us for the implicit
  // GEMM's 256 x 64 tiles).
  if (forced <= 0) {
    if (c.C_in == 64 && c.K == 64 && c.u == 1 && c.v == 1 && eb == 2 && aligned(c.x, 16) &&
        aligned(c.w, 16) && c.H * c.W * 128 < (int64_t(1) << 31)) {
      const int rc = launch_conv_slab(p, c.type, stream);
      if (rc != TLA_ERR_UNSUPPORTED || forced == 0) return rc;
    } else if (forced == 0) {
      return TLA_ERR_UNSUPPORTED;
    }
  }
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
  // -> 256 two stages measured 45.4 us against 52.8 us for three.  The
  // 256 x 64 tile runs 8 wavefronts (4 x 2 of 64 x 32): each thread issues
  // half the copies of the 4-wavefront form, and a wave blocked on a copy
  // leaves its SIMD to the other wave's MFMAs (17.8 against 18.5 us).
  if (forced == 1 && !fast) return TLA_ERR_UNSUPPORTED;
  if (fast && forced != 2) {
    const bool narrow = c.K <= 64;
    if (c.type == TLA_BF16)
      return narrow ? launch_fast<kBF16, 256, 64, 128, 2, 1, 4, 2, true>(p, stream)
                    : launch_fast<kBF16, 128, 128, 128, 2, 1, 2, 2, true>(p, stream);
    return narrow ? launch_fast<kF16, 256, 64, 128, 2, 1, 4, 2, true>(p, stream)
                  : launch_fast<kF16, 128, 128, 128, 2, 1, 2, 2, true>(p, stream);
  }
  return launch_conv_general(p, c.type, stream);
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
  if (g.C && ceb == 2 && g.c_order == TLA_ROW_MAJOR && aligned(g.C, 2)) p.flags |= kC2;
  if (g.d_order == TLA_ROW_MAJOR && aligned(g.D, 2)) p.flags |= kD2;
  if (g.bias && aligned(g.bias, 4 * beb)) p.flags |= kBiasVec;
  const bool a_vec = (g.a_order == TLA_ROW_MAJOR) && ((g.lda * eb) % 16 == 0) && aligned(g.A, 16);
  const bool b_rows16 = ((g.ldb * eb) % 16 == 0) && aligned(g.B, 16);
  const bool b_vec = (g.b_order == TLA_COL_MAJOR) && b_rows16;
  // 16-bit N-contiguous B (the general kernel reads it by rows of n)
  const bool nt = eb == 2 && g.b_order == TLA_ROW_MAJOR;
  // bit 9: B's contiguous runs (K runs, or N runs when nt) are 16-byte aligned
  p.flags |= (a_vec ? 1 << 8 : 0) | ((b_vec || (nt && b_rows16)) ? 1 << 9 : 0);
  const int BK = fast_slab_bytes(g.a_type) / eb;
  // the fast kernel addresses each operand with 32-bit offsets below 2^31
  const bool small_ops = (int64_t)g.M * g.lda * eb < (int64_t(1) << 31) &&
                         (int64_t)g.N * g.ldb * eb < (int64_t(1) << 31);
  // K: any multiple of the 16-byte chunk -- the last k-tile's chunks past K
  // read zeros (e4m3 off the 128-byte slab: the two-group kernel only)
  const bool k_ok = g.K > 0 && (g.K % (16 / eb)) == 0;
  const bool k_slab = g.K > 0 && (g.K % BK) == 0;
  const bool fast = a_vec && b_vec && small_ops && k_ok;
  // A in the fast layout, B a 16-bit row-major K x N matrix with 16-byte
  // aligned rows and whole 16-byte chunks of columns, below 2 GiB
  const bool bt = !fast && nt && a_vec && b_rows16 && g.N % 8 == 0 &&
                  (int64_t)g.M * g.lda * eb < (int64_t(1) << 31) &&
                  (int64_t)g.K * g.ldb * eb < (int64_t(1) << 31) && k_ok;
  // A a 16-bit column-major M x K matrix with 16-byte aligned columns, M a
  // multiple of 8, below 2 GiB; B K-contiguous or N-contiguous as above
  const bool b_any = (b_vec && (int64_t)g.N * g.ldb * eb < (int64_t(1) << 31)) ||
                     (nt && b_rows16 && g.N % 8 == 0 &&
                      (int64_t)g.K * g.ldb * eb < (int64_t(1) << 31));
  const bool at = eb == 2 && g.a_order == TLA_COL_MAJOR && ((g.lda * eb) % 16) == 0 &&
                  aligned(g.A, 16) && g.M % 8 == 0 &&
                  (int64_t)g.K * g.lda * eb < (int64_t(1) << 31) && k_ok && b_any;
  const int64_t tiles256 = ((g.M + 255) / 256) * ((g.N + 255) / 256);
  const bool big = tiles256 >= 128;
  switch (g.a_type) {
    case TLA_BF16:
      return dispatch_typed<kBF16>(p, fast, bt, at, big, k_slab, stream, dry_run, name, forced);
    case TLA_F16:
      return dispatch_typed<kF16>(p, fast, bt, at, big, k_slab, stream, dry_run, name, forced);
    case TLA_E4M3:
      return dispatch_typed<kE4M3>(p, fast, false, false, big, k_slab, stream, dry_run, name,
                                   forced);
    default: return TLA_ERR_UNSUPPORTED;
  }
}

}  // namespace tla
