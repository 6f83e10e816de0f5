// gemm_general.hip -- the four-wavefront GEMM kernel (2 x 2 waves of
// (BM/2) x (BN/2), two LDS stages) for gfx950, in two forms:
//
//   register-staged  the general path: any order, pitch or alignment of A
//                    and B, ragged K.  Each thread loads its chunks of a
//                    k-tile into registers before the MFMAs of an earlier
//                    one (two tiles ahead inside K) and writes them to the
//                    other LDS stage after the MFMAs of the tile before it.
//                    Elements outside the matrix load as zero.  Also the
//                    implicit-GEMM convolution's fallback loader.
//   direct-to-LDS    e4m3 in the fast layout (variants 1 and 3).
//
//   D = act(alpha_eff * A.B + beta*C + bias),  fp32 accumulation.
//
// The tiling follows "CUTLASS / CuTe 主线" (hpc.payai.win/cutlass), section
// 一: a workgroup owns a BM x BN block tile of D, each wavefront a quarter of
// it, each 32x32 MFMA a 32x32 piece of that.  The epilogue is the shared
// one of gemm_common.hpp.
#include "gemm_common.hpp"

namespace tla {
namespace {

// ------------------------------------------------------------------ kernel
// kStages LDS stages of BM + BN rows of kRowBytes bytes each.  K-tile kt
// lives in stage kt % kStages; up to kStages - 1 tiles are in flight, so the
// copy of a tile has kStages - 1 tiles of matrix-core work to arrive in.
//
// Register-staged operand views (fixed per instantiation, so the loader
// carries no stride it does not use): kAKC, A is K-contiguous (row-major),
// else M-contiguous -- 16-bit A then has its slab as k rows of m
// (RegSlabNT), e4m3 A goes through element loads; kBView: B K-contiguous
// (kBK), N-contiguous through element loads (kBN), or N-contiguous 16-bit
// with its slab as k rows of n (RegSlabNT, kBNT).  A k-rows slab is read
// into fragments by transposing LDS reads.  kT8: an e4m3 operand that is M-
// or N-contiguous with 16-byte aligned runs is loaded by RegSlabT8 instead
// of element loads.
enum : int { kBK = 0, kBN = 1, kBNT = 2 };

// An 8-bit operand stored with its rows of m (or n) contiguous -- a column-
// major A or a row-major B -- whose runs are 16-byte aligned.  Thread t
// loads the 16-byte runs of rows 16 (t % 8) .. + 15 at the four k indices
// 4 (t / 8) .. + 3, transposes the 4 x 16 bytes in registers and writes 16
// dwords of four consecutive k each, so the slab holds the tile as rows of
// k (swizzled 16-byte chunks), as the K-contiguous loader leaves it, and the
// fragment reads do not change.  One 128-row by 128-byte tile per 256
// threads.  Indices k past K load as zero and so do rows past the edge; the
// run that crosses the edge is gathered byte by byte, clamped in bounds.
template <int ROWS, int kRowBytes>
struct RegSlabT8 {
  using Swz = typename Slab<kRowBytes>::Swz;
  static_assert(ROWS == 128 && kRowBytes == 128 && kThreads == 256,
                "128 x 128-byte tile on 256 threads");
  i32x4 v[4];

  // k0 .. k0 + 127 inside K, rows row0 .. row0 + 127 inside rows_valid;
  // s: the k stride in elements (a multiple of 16, base 16-byte aligned)
  __device__ __forceinline__ void load_whole(const uint8_t* __restrict__ base, int64_t s, int row0,
                                             int rows_valid, int k0, int tid) {
    const uint8_t* q = base + (int64_t)(k0 + 4 * (tid >> 3)) * s + row0 + 16 * (tid & 7);
#pragma unroll
    for (int it = 0; it < 4; ++it) v[it] = *(const i32x4*)(q + it * s);
  }

  __device__ __forceinline__ void load_edge(const uint8_t* __restrict__ base, int64_t s, int row0,
                                            int rows_valid, int k0, int K, int tid) {
    const int c = row0 + 16 * (tid & 7);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int k = k0 + 4 * (tid >> 3) + it;
      i32x4 x = {0, 0, 0, 0};
      if (k < K && c < rows_valid) {
        const uint8_t* row = base + (int64_t)k * s;
        if (c + 16 <= rows_valid)
          x = *(const i32x4*)(row + c);
        else
          x = gather16<1>(row, 1, c, rows_valid, rows_valid - 1);
      }
      v[it] = x;
    }
  }

  __device__ __forceinline__ void store(uint8_t* slab, int tid) const {
    const int kk = 4 * (tid >> 3), r0 = 16 * (tid & 7);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t x0 = v[0][d], x1 = v[1][d], x2 = v[2][d], x3 = v[3][d];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t y = ((x0 >> (8 * b)) & 0xffu) | (((x1 >> (8 * b)) & 0xffu) << 8) |
                           (((x2 >> (8 * b)) & 0xffu) << 16) | (((x3 >> (8 * b)) & 0xffu) << 24);
        const int r = r0 + 4 * d + b;
        *(uint32_t*)(slab + r * kRowBytes + Swz::chunk(r, kk >> 4) * 16 + (kk & 15)) = y;
      }
    }
  }
};

// The register-staged form without element-wise views asks for two waves
// per SIMD (at most 256 VGPRs): left to itself the compiler let its two
// register sets push the kernel to 260-316 VGPRs, one wave per SIMD.  With
// an element-wise view it would spill, so those keep one.
template <int kCode, int BM, int BN, int kRowBytes, int kStages, bool kFast, bool kConv = false,
          bool kAKC = true, int kBView = kBK, bool kT8 = false>
__global__ __launch_bounds__(kThreads, (kFast || (!kAKC && elem_bytes(kCode) != 2) ||
                                        kBView == kBN) ? 1 : 2) void gemm_kernel(const GemmParams p) {
  constexpr bool kNT = kBView == kBNT;
  constexpr bool kAT = !kAKC && elem_bytes(kCode) == 2;  // A as k rows of m
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
  static_assert(!kNT || (EB == 2 && Atom::kK == 16 && !kFast && !kConv),
                "N-contiguous B slab: 16-bit operands, register-staged path");
  static_assert(!(kFast || kConv) || (kAKC && kBView == kBK), "K-contiguous operands");
  static_assert(!kT8 || (EB == 1 && BM == 128 && BN == 128 && kRowBytes == 128 && !kFast &&
                         (!kAKC || kBView == kBN)), "8-bit runs along M or N");
  constexpr bool kA8 = kT8 && !kAKC, kB8 = kT8 && kBView == kBN;
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
      if constexpr (kAT)
        a[buf][i] = load_frag_nt<2 * BM>(stage, wm0 + 32 * i, ks, lane);
      else
        a[buf][i] = load_frag<kCode, kRowBytes>(stage, wm0 + 32 * i + (lane & 31), ks, lane);
    });
    static_for<FN>([&](auto j) {
      if constexpr (kNT)
        b[buf][j] = load_frag_nt<2 * BN>(stage + SLAB_A, wn0 + 32 * j, ks, lane);
      else
        b[buf][j] = load_frag<kCode, kRowBytes>(stage + SLAB_A, wn0 + 32 * j + (lane & 31), ks,
                                                lane);
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
    // Two register sets per operand.  Tiles 0 .. KTw - 1 lie inside K; they
    // load as whole chunks with no per-lane branch, two tiles ahead: tile
    // t + 2 goes into set t % 2 before the MFMAs of tile t, and set
    // (t + 1) % 2 (tile t + 1, loaded a whole iteration earlier) is written
    // to the other LDS stage after them.  The ragged rest goes one tile
    // ahead through the edge loader.  Tile t lives in LDS stage t % 2.
    using RA = std::conditional_t<
        kConv, ConvSlab<BM, EB, kRowBytes>,
        std::conditional_t<kAT, RegSlabNT<BM, BK>,
                           std::conditional_t<kA8, RegSlabT8<BM, kRowBytes>,
                                              RegSlab<BM, EB, kRowBytes, kAKC>>>>;
    using RB = std::conditional_t<
        kNT, RegSlabNT<BN, BK>,
        std::conditional_t<kB8, RegSlabT8<BN, kRowBytes>, RegSlab<BN, EB, kRowBytes, kBView == kBK>>>;
    RA ra[2];
    RB rb[2];
    const bool a_vec = (p.flags >> 8) & 1;
    const int64_t a_s = kAKC ? p.a_sr : p.a_sk;  // the stride that is not 1
    const int64_t b_s = kBView == kBK ? p.b_sr : p.b_sk;
    auto load = [&](int k0, auto whole, auto set) {
      if constexpr (kConv) {
        ra[set].load_conv(p, m0, k0, a_vec, tid);
      } else {
        if constexpr (kAT || kA8) {
          if constexpr (whole) ra[set].load_whole(p.A, a_s, m0, p.M, k0, tid);
          else ra[set].load_edge(p.A, a_s, m0, p.M, k0, p.K, tid);
        } else {
          if constexpr (whole && kAKC) ra[set].load_whole(p.A, a_s, m0, p.M, k0, tid);
          else ra[set].load_edge(p.A, a_s, m0, p.M, k0, p.K, tid);
        }
      }
      if constexpr (kNT || kB8) {
        if constexpr (whole) rb[set].load_whole(p.B, b_s, n0, p.N, k0, tid);
        else rb[set].load_edge(p.B, b_s, n0, p.N, k0, p.K, tid);
      } else {
        if constexpr (whole && kBView == kBK) rb[set].load_whole(p.B, b_s, n0, p.N, k0, tid);
        else rb[set].load_edge(p.B, b_s, n0, p.N, k0, p.K, tid);
      }
    };
    auto store = [&](uint8_t* st, auto set) {
      ra[set].store(st, tid);
      rb[set].store(st + SLAB_A, tid);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using Whole = std::true_type;
    using Edge = std::false_type;
    // whole tiles: inside K; for a k-rows slab of a tile that crosses M or N
    // also before the tile holding row K - 1 (its chunks read past the edge)
    const bool m_edge = kAT && m0 + BM > p.M, n_edge = kNT && n0 + BN > p.N;
    // (the 8-bit runs loader has no clamped whole load: its edge tiles take
    // the edge loop throughout)
    const bool t8_edge = (kA8 && m0 + BM > p.M) || (kB8 && n0 + BN > p.N);
    const int KTw = t8_edge ? 0
                    : (m_edge || n_edge)
                        ? ((m_edge && p.M < 8) || (n_edge && p.N < 8) ? 0 : (p.K - 1) / BK)
                        : p.K / BK;
    if (KT > 0) {
      if (KTw > 0) load(0, Whole{}, S0{});
      else load(0, Edge{}, S0{});
      store(smem, S0{});
      if (KTw > 1) load(BK, Whole{}, S1{});
    }
    __syncthreads();
    // the MFMAs of tile kt between two scheduling fences: the loads before
    // them, the LDS writes (which wait for loads) after them
    auto fenced_compute = [&](int kt) {
      __builtin_amdgcn_sched_barrier(0);
      compute(smem + (kt & 1) * STAGE);
      __builtin_amdgcn_sched_barrier(0);
    };
    // whole tile kt in stage S, tile kt + 1 in set S ^ 1: load tile kt + 2
    // (clamped to the last whole tile, so the load count never varies) into
    // set S, multiply, write set S ^ 1 to the other stage
    auto whole_step = [&](int kt, auto S) {
      constexpr int kO = S ^ 1;
      load(min(kt + 2, KTw - 1) * BK, Whole{}, S);
      fenced_compute(kt);
      store(smem + kO * STAGE, std::integral_constant<int, kO>{});
      __syncthreads();
    };
    int kt = 0;
    for (; kt + 2 < KTw; kt += 2) {
      whole_step(kt, S0{});
      whole_step(kt + 1, S1{});
    }
    if (kt + 1 < KTw) {  // tile kt + 1 is whole and already in set 1
      fenced_compute(kt);
      store(smem + STAGE, S1{});
      __syncthreads();
      ++kt;
    }
    for (; kt + 1 < KT; ++kt) {  // the ragged rest, one tile ahead in set 0
      load((kt + 1) * BK, Edge{}, S0{});
      fenced_compute(kt);
      store(smem + ((kt + 1) & 1) * STAGE, S0{});
      __syncthreads();
    }
    if (kt < KT) compute(smem + (kt & 1) * STAGE);
  }

  // Epilogue: acc[i][j] holds the D^T piece for rows m0+wm0+32i.. and
  // columns n0+wn0+32j..; value r of lane l sits at (row, col) =
  // (lane%32, mfma32_acc_row(l, r)) of that 32x32 piece.  No copy is in
  // flight here; after the barrier the stages are the waves' regions.
  constexpr bool kLdsEpi = 4 * WM * 64 * FN <= kStages * STAGE;
  __syncthreads();
  epilogue_tiles<FM, FN, !kFast>(p, m0 + wm0, n0 + wn0, lane, acc,
                         kLdsEpi ? smem + wave * WM * 64 * FN : nullptr);
}


template <int kCode, int BM, int BN, bool kFast, bool kConv, bool kAKC, int kBView,
          bool kT8 = false>
int launch(const GemmParams& p0, hipStream_t stream) {
  GemmParams p = p0;
  int64_t grid;
  set_grid(p, BM, BN, &grid);
  if (grid <= 0) return TLA_OK;
  if (grid > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((gemm_kernel<kCode, BM, BN, 128, 2, kFast, kConv, kAKC, kBView, kT8>),
                     dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
}

// The register-staged kernel for the operand views p's strides describe
// (A: a_sk == 1 K-contiguous, else M-contiguous; B: b_sk == 1 K-contiguous,
// else N-contiguous, which 16-bit operands take through the k-rows-of-n
// slab).  3001 x 4097 x 777 fp16 with A and B row-major at odd pitches:
// 167 us with B's slab as k rows of n, 738 us with n rows of k filled element
// by element.
template <int kCode>
int launch_views(const GemmParams& p, hipStream_t s) {
  constexpr int kBNc = kCode == kE4M3 ? kBN : kBNT;
  const bool akc = p.a_sk == 1, bkc = p.b_sk == 1;
  if constexpr (kCode == kE4M3) {
    // M- or N-contiguous e4m3 operands with 16-byte aligned runs: RegSlabT8
    // (4096^3 with both operands column-major: 1130 us with element loads)
    auto runs16 = [](const void* q, int64_t ld) {
      return (reinterpret_cast<uintptr_t>(q) & 15) == 0 && ld % 16 == 0;
    };
    if ((!akc || !bkc) && (akc || runs16(p.A, p.a_sk)) && (bkc || runs16(p.B, p.b_sk))) {
      if (akc) return launch<kCode, 128, 128, false, false, true, kBN, true>(p, s);
      return bkc ? launch<kCode, 128, 128, false, false, false, kBK, true>(p, s)
                 : launch<kCode, 128, 128, false, false, false, kBN, true>(p, s);
    }
  }
  if (akc)
    return bkc ? launch<kCode, 128, 128, false, false, true, kBK>(p, s)
               : launch<kCode, 128, 128, false, false, true, kBNc>(p, s);
  return bkc ? launch<kCode, 128, 128, false, false, false, kBK>(p, s)
             : launch<kCode, 128, 128, false, false, false, kBNc>(p, s);
}

}  // namespace

int launch_general(const GemmParams& p, int type, hipStream_t stream) {
  switch (type) {
    case kBF16: return launch_views<kBF16>(p, stream);
    case kF16: return launch_views<kF16>(p, stream);
    case kE4M3: return launch_views<kE4M3>(p, stream);
    default: return TLA_ERR_UNSUPPORTED;
  }
}

int launch_two_stage_e4m3(const GemmParams& p, bool big, hipStream_t stream) {
  return big ? launch<kE4M3, 256, 256, true, false, true, kBK>(p, stream)
             : launch<kE4M3, 128, 128, true, false, true, kBK>(p, stream);
}

int launch_conv_general(const GemmParams& p, int type, hipStream_t stream) {
  switch (type) {
    case kBF16: return launch<kBF16, 128, 128, false, true, true, kBK>(p, stream);
    case kF16: return launch<kF16, 128, 128, false, true, true, kBK>(p, stream);
    default: return TLA_ERR_UNSUPPORTED;
  }
}

const void* general_kernel(int type) {
  switch (type) {
    case kBF16: return (const void*)gemm_kernel<kBF16, 128, 128, 128, 2, false>;
    case kF16: return (const void*)gemm_kernel<kF16, 128, 128, 128, 2, false>;
    case kE4M3: return (const void*)gemm_kernel<kE4M3, 128, 128, 128, 2, false>;
    default: return nullptr;
  }
}

const void* two_stage_e4m3_kernel(bool big) {
  return big ? (const void*)gemm_kernel<kE4M3, 256, 256, 128, 2, true>
             : (const void*)gemm_kernel<kE4M3, 128, 128, 128, 2, true>;
}

}  // namespace tla
