// conv_slab.hip -- forward convolution with 64 input and 64 output channels
// at stride 1, computed from an image slab and the whole filter held in LDS.
//
//   y[n, p, q, k] = act(alpha * sum_{r,s,c} x[n, p - ph + r*dh, q - pw + s*dw, c] * w[k, r, s, c]
//                       + beta * C[n, p, q, k] + bias[k])
//
// The implicit GEMM of the PitchLinearStripminedThreadMap walk-through
// (section 5.2: one GEMM dimension is the output pixel, the other the filter
// tap times the input channel) gathers each row of A from the image, so a
// tiled mainloop copies every image element into LDS once per filter tap.
// With 64 channels that copy traffic, not the matrix cores, bounds the layer.
// Here a workgroup owns RW whole output rows of one image (RW*Q pixels, at
// most 512) and all 64 output channels:
//
//   * LDS holds the filter (R*S taps x 64 output channels x 128 bytes) and
//     the image slab those rows read (RW + (R-1)*dh input rows of
//     Q + (S-1)*dw pixels, zero outside the image), each copied in once;
//   * the slab stores a pixel's 128 bytes of channels at a 144-byte stride,
//     so the 32 consecutive pixels of an A fragment fall into distinct LDS
//     banks and a filter tap is a uniform offset; the filter's 16-byte chunks
//     are XOR-swizzled by output channel for the same reason;
//   * each of the 8 wavefronts multiplies 64 consecutive pixels (two groups
//     of 32) by both 32-channel halves of the filter: per k step (one tap, 16
//     channels) it reads two filter fragments and two pixel fragments and
//     issues four 32x32x16 MFMAs, with the reads two steps ahead;
//   * the epilogue is the GEMM's (alpha, beta*C, bias, activation) on the
//     wave's 64 x 64 tile, staged through LDS once the slab is done with.
//
// Both fills are direct HBM -> LDS copies that land lane-linearly; each lane
// works out which image pixel (or filter chunk) its 16 bytes are, and lanes
// that fall on the slab's pixel padding or outside the image get an offset
// past the buffer's record count, which reads zeros.
#include "gemm_common.hpp"

namespace tla {
namespace {

constexpr int kWaves = 8;
constexpr int kGroups = 2;                 // pixel groups of 32 per wavefront
constexpr int kRound = 1024 * kWaves;      // LDS bytes one copy round fills
constexpr int kSlabLds = 160 * 1024;       // the whole LDS of a CU
constexpr int kPixStride = 144;            // bytes per slab pixel (128 of channels)
constexpr int kFilterTap = 64 * 128;       // filter bytes per tap
constexpr int kMaxPix = 32 * kGroups * kWaves;

// The epilogue of a wave tile whose first `valid` rows (of 32 * kGroups) are
// output pixels: C (16-bit, rows of 64 channels) comes into the wave's LDS
// region with whole-row copies, the 16-bit result goes back in place and
// leaves as whole rows, as in the full-tile LDS epilogue; copies and stores
// of rows past `valid` are predicated off.  The region's 16-byte chunks are
// XOR-swizzled by row so that the row-per-lane accesses of one instruction
// fall into distinct banks.
template <int kAct, bool kBf16, bool kHasC>
__device__ __forceinline__ void epilogue_rows(const GemmParams& p, int m_base, int valid, int lane,
                                              const f32x16 (&acc)[kGroups][2], uint8_t* region) {
  constexpr int kRowB = 128, kCh = 8, kRowsPerKiB = 8, kIters = 32 * kGroups * kRowB / 1024;
  auto swz = [](int r, int c) { return c ^ ((r >> 1) & (kCh - 1)); };
  const int row = lane & 31, half = lane >> 5;
  const int rr = lane / kCh, cs = lane % kCh;  // row-wise view of one KiB
  if constexpr (kHasC) {
    const uint8_t* C = p.C + (int64_t)m_base * 128;
    static_for<kIters>([&](auto t) {
      const int r = kRowsPerKiB * t + rr;
      if (r < valid)
        __builtin_amdgcn_global_load_lds(C + r * 128 + swz(r, cs) * 16, to_lds(region + t * 1024),
                                         16, 0, 0);
    });
  }
  uint2 braw[2][4];
  load_bias16<2>(p, 0, half, braw);
  wait_vmcnt<0>();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  static_for<kGroups>([&](auto i) {
    static_for<2>([&](auto j) {
      static_for<4>([&](auto g) {
        const int r = 32 * i + row;
        uint8_t* slot = region + r * kRowB + swz(r, 4 * j + g) * 16 + 8 * half;
        const uint2 c = kHasC ? *(const uint2*)slot : uint2{0u, 0u};
        *(uint2*)slot = epi_group<kAct, kBf16, kHasC>(acc[i][j], g, c, braw[j][g], p.alpha, p.beta);
      });
    });
  });
  uint8_t* D = p.D + (int64_t)m_base * 128;
  static_for<kIters>([&](auto t) {
    const int r = kRowsPerKiB * t + rr;
    const i32x4 v = *(const i32x4*)(region + t * 1024 + lane * 16);
    if (r < valid) *(i32x4*)(D + r * 128 + swz(r, cs) * 16) = v;
  });
}

template <int kAct, bool kBf16>
__device__ __forceinline__ void epilogue_rows_c(const GemmParams& p, int m_base, int valid, int lane,
                                                const f32x16 (&acc)[kGroups][2], uint8_t* region) {
  if (p.beta != 0.f) epilogue_rows<kAct, kBf16, true>(p, m_base, valid, lane, acc, region);
  else epilogue_rows<kAct, kBf16, false>(p, m_base, valid, lane, acc, region);
}

template <bool kBf16>
__device__ __forceinline__ void epilogue_rows_t(const GemmParams& p, int m_base, int valid, int lane,
                                                const f32x16 (&acc)[kGroups][2], uint8_t* region) {
  switch (p.act) {
    case TLA_ACT_RELU:
      epilogue_rows_c<TLA_ACT_RELU, kBf16>(p, m_base, valid, lane, acc, region);
      break;
    case TLA_ACT_GELU:
      epilogue_rows_c<TLA_ACT_GELU, kBf16>(p, m_base, valid, lane, acc, region);
      break;
    default:
      epilogue_rows_c<TLA_ACT_NONE, kBf16>(p, m_base, valid, lane, acc, region);
      break;
  }
}

__device__ __forceinline__ void epilogue_rows_switch(const GemmParams& p, int m_base, int valid,
                                                     int lane, const f32x16 (&acc)[kGroups][2],
                                                     uint8_t* region) {
  if (p.d_type == kBF16) epilogue_rows_t<true>(p, m_base, valid, lane, acc, region);
  else epilogue_rows_t<false>(p, m_base, valid, lane, acc, region);
}

template <int kCode>
__global__ __launch_bounds__(64 * kWaves) void conv_slab_kernel(const GemmParams p, int RW, int SW,
                                                                int SR, int w_region,
                                                                int slab_rounds, int rows_per_image,
                                                                uint32_t sw_magic) {
  static_assert(kRound % kFilterTap == 0, "a copy round covers whole filter taps");
  using Atom = MfmaAtom<kCode>;
  using Frag = typename Atom::Frag;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSlabLds];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = blockIdx.x / rows_per_image;
  const int h0 = (blockIdx.x - n * rows_per_image) * RW;   // first output row
  const int H = p.cH, W = p.cW, Q = p.cQ, S = p.cS, RS = p.cR * S;
  const int rows = min(RW, p.cP - h0);
  const int npix = rows * Q;                               // valid pixels
  const int m0 = (n * p.cP + h0) * Q;                      // first output pixel

  // ---- copies.  Filter round i fills LDS bytes [kRound i, kRound (i + 1)):
  // thread t the 16 bytes at kRound i + 16 t = (tap, output channel k, chunk
  // position), fetched from chunk position ^ swizzle(k) of w[k, tap]; taps
  // past the last read zeros (the filter region is whole rounds).
  // Slab round i fills bytes [8192 i, ..) of the slab region, whose byte o
  // is byte o % 144 of slab pixel o / 144 (slab row hs = pixel / SW, column
  // ws; bytes 128..143 of a pixel are padding); sw_magic = ceil(2^31 / SW)
  // turns the division by SW into a high multiply of 2 * pixel, exact for
  // the slab's pixel counts (below 2^11).
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.B, 0, RS * kFilterTap, 0x00020000);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.A + (int64_t)n * H * W * 128), 0, H * W * 128, 0x00020000);
  const int wk = (tid >> 3) & 63, wpos = tid & 7, wtap = tid >> 9;
  const uint32_t wsrc = (uint32_t)((wk * RS * 8 + (wpos ^ ((wk >> 1) & 7))) * 16);
  auto copy_filter = [&](int i) {
    const int tap = i * (kRound / kFilterTap) + wtap;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        wr, (__attribute__((address_space(3))) void*)(smem + i * kRound + wave * 1024), 16,
        tap < RS ? wsrc + tap * 128 : 0x80000000u, 0, 0, 0);
  };
  const int hb = h0 - p.cph;                               // image row of slab row 0
  auto copy_slab = [&](int i) {
    const int o = i * kRound + tid * 16;
    const int pix = o / kPixStride, sb = o - pix * kPixStride;
    const int hs = (int)__umulhi((uint32_t)pix << 1, sw_magic), ws = pix - hs * SW;
    const int h = hb + hs, w = ws - p.cpw;
    const bool ok = sb < 128 && hs < SR && h >= 0 && h < H && w >= 0 && w < W;
    const uint32_t src = ok ? (uint32_t)((h * W + w) * 128 + sb) : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        xr, (__attribute__((address_space(3))) void*)(smem + w_region + i * kRound + wave * 1024),
        16, src, 0, 0, 0);
  };
  for (int i = 0; i < w_region / kRound; ++i) copy_filter(i);
  for (int i = 0; i < slab_rounds; ++i) copy_slab(i);
  wait_vmcnt<0>();
  stage_barrier();

  // ---- fragment addresses.  Wave v owns pixels 64 v .. 64 v + 63 of the
  // workgroup, its group g pixels 64 v + 32 g ..; pixels past the valid ones
  // read the last valid pixel (their results are not stored).
  const int half = lane >> 5;
  const bool busy = kGroups * 32 * wave < npix;
  f32x16 acc[kGroups][2];
  if (busy) {
    uint32_t abase[kGroups];
    static_for<kGroups>([&](auto g) {
      const int px = min(32 * (kGroups * wave + (int)g) + (lane & 31), npix - 1);
      const int oh = px / Q, oq = px - oh * Q;
      abase[g] = (uint32_t)(w_region + (oh * SW + oq) * kPixStride + half * 16);
    });
    // filter fragment of output channels 32 j + lane % 32, chunk 2 kk + half
    uint32_t bbase[4];
    static_for<4>([&](auto kk) {
      const int k = lane & 31;
      bbase[kk] = (uint32_t)(k * 128 + ((2 * kk + half) ^ ((k >> 1) & 7)) * 16);
    });
    static_for<kGroups>([&](auto g) { acc[g][0] = f32x16{}; acc[g][1] = f32x16{}; });
    // four register sets, one per kk: the reads of a step go out two steps
    // ahead of its MFMAs
    Frag fa[4][kGroups], fb[4][2];
    // k step (tap, kk): filter bytes at tap * 8192, slab bytes at the tap's
    // pixel offset; kk selects 16 channels
    auto read_step = [&](auto buf, int tap, int toff, auto kk) {
      static_for<2>([&](auto j) {
        fb[buf][j] = *(const Frag*)(smem + bbase[kk] + tap * kFilterTap + j * 4096);
      });
      static_for<kGroups>([&](auto g) {
        fa[buf][g] = *(const Frag*)(smem + abase[g] + toff + kk * 32);
      });
    };
    auto mma_step = [&](auto buf) {
      static_for<kGroups>([&](auto g) {
        static_for<2>([&](auto j) { Atom::mma(acc[g][j], fb[buf][j], fa[buf][g]); });
      });
    };
    // slab offset of tap (r, s) = (r dh SW + s dw) * 144, stepped per tap
    const int step_s = p.cdw * kPixStride;
    const int step_r = (p.cdh * SW - (S - 1) * p.cdw) * kPixStride;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // the two steps' reads in step order, so that the loop's waits (which
    // assume that order from the previous iteration) stay exact on entry
    __builtin_amdgcn_sched_barrier(0);
    read_step(I0{}, 0, 0, I0{});
    __builtin_amdgcn_sched_barrier(0);
    read_step(I1{}, 0, 0, I1{});
    int toff = 0, s_tap = 0;
    for (int tap = 0; tap < RS; ++tap) {
      // the last tap's prefetches re-read it (unused)
      const int nt = tap + 1 < RS ? tap + 1 : tap;
      const int ntoff = tap + 1 < RS ? toff + (s_tap + 1 < S ? step_s : step_r) : toff;
      static_for<4>([&](auto kk) {
        constexpr int ahead = (kk + 2) & 3;
        using IA = std::integral_constant<int, ahead>;
        // step kk + 2's reads go out before step kk's MFMAs, fenced so that
        // the scheduler neither sinks them next to their first use nor lets
        // the register sets share registers; the MFMAs then wait only for
        // the fragments read two steps earlier
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kk < 2)
          read_step(IA{}, tap, toff, IA{});
        else
          read_step(IA{}, nt, ntoff, IA{});
        __builtin_amdgcn_sched_barrier(0);
        mma_step(std::integral_constant<int, (int)kk>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      toff = ntoff;
      s_tap = s_tap + 1 < S ? s_tap + 1 : 0;
    }
  }

  // ---- epilogue of the wave's tile.  Once every wave is done with the slab
  // and the filter, each wave stages its tile's C and y through its own
  // LDS region, so both move as whole rows; rows past the workgroup's valid
  // pixels are left alone.  (The release fence keeps every slab and filter
  // read of this wave above the barrier: the regions overlap them.)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  stage_barrier();
  if (!busy) return;
  GemmParams e = p;
  e.M = m0 + npix;
  const int m_base = m0 + 32 * kGroups * wave;
  const int valid = min(32 * kGroups, npix - 32 * kGroups * wave);
  uint8_t* region = smem + wave * (32 * kGroups * 128);
  const bool b_ok = !p.bias || ((p.flags & kBiasVec) && p.bias_type == p.d_type);
  const bool c_ok = p.beta == 0.f || (p.c_type == p.d_type && (p.flags & kC16));
  if (valid < 32 * kGroups && b_ok && c_ok && (p.flags & kD16))
    epilogue_rows_switch(e, m_base, valid, lane, acc, region);
  else
    epilogue_tiles<kGroups, 2>(e, m_base, 0, lane, acc, region);
}

}  // namespace

// Rows per workgroup: each workgroup costs about the same (every busy
// wavefront multiplies two whole pixel groups; the slab copy grows only by
// RW rows in RW + R - 1), so the time is set by the launch rounds of 256
// workgroups, and among the fewest rounds the smallest RW spreads the
// pixels over the most workgroups and copies the least slab per workgroup.
// On 32 x 56 x 56 x 64 -> 64 (3x3) RW = 7 (256 workgroups) measured
// 14.7 us against 13.8-15.8 for RW = 8 (224) and 23 for RW = 4 (448).
int launch_conv_slab(const GemmParams& p, int type, hipStream_t stream) {
  const int RS = p.cR * p.cS, Q = p.cQ, P = p.cP, N = p.M / (P * Q);
  const int SW = Q + (p.cS - 1) * p.cdw;
  const int64_t w_region = ((int64_t)kFilterTap * RS + kRound - 1) / kRound * kRound;
  int best = 0;
  int64_t best_rounds = 0;
  for (int rw = 1; rw * Q <= kMaxPix && rw <= P; ++rw) {
    const int64_t sr = rw + (int64_t)(p.cR - 1) * p.cdh;
    const int64_t slab = (sr * SW * kPixStride + kRound - 1) / kRound * kRound;
    if (w_region + slab > kSlabLds) break;
    const int64_t rounds = ((int64_t)N * ((P + rw - 1) / rw) + 255) / 256;
    if (best == 0 || rounds < best_rounds) { best = rw; best_rounds = rounds; }
  }
  if (best == 0) return TLA_ERR_UNSUPPORTED;
  const int RW = best, SR = RW + (p.cR - 1) * p.cdh;
  const int slab_rounds = (SR * SW * kPixStride + kRound - 1) / kRound;
  const int rows_per_image = (P + RW - 1) / RW;
  const uint32_t sw_magic = (uint32_t)(((uint64_t(1) << 31) + SW - 1) / SW);
  const int64_t grid = (int64_t)N * rows_per_image;
  if (grid <= 0) return TLA_OK;
  if (grid > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
  if (type == TLA_BF16)
    hipLaunchKernelGGL(conv_slab_kernel<kBF16>, dim3((unsigned)grid), dim3(64 * kWaves), 0, stream,
                       p, RW, SW, SR, (int)w_region, slab_rounds, rows_per_image, sw_magic);
  else
    hipLaunchKernelGGL(conv_slab_kernel<kF16>, dim3((unsigned)grid), dim3(64 * kWaves), 0, stream,
                       p, RW, SW, SR, (int)w_region, slab_rounds, rows_per_image, sw_magic);
  return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
}

}  // namespace tla
