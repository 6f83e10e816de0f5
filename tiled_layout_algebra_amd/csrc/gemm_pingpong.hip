// gemm_pingpong.hip -- the 256 x 256 block-tile GEMM with two wavefront
// groups that take turns on the matrix cores.
//
// Tiling (the three levels of "CUTLASS / CuTe 主线", section 一): a
// workgroup owns a 256 x 256 tile of D; its eight 64-lane wavefronts form two
// groups of four, group g owning rows 128g .. 128g+127 of the tile; inside a
// group the four waves split those rows 2 x 2 into 64 x 128 wave tiles;
// under a wave tile sit 2 x 4 MFMA 32x32 instruction tiles.  A K step
// (section 二's mainloop) moves one 128-byte-wide K slab of A and of B
// (64 bf16/fp16 or 128 e4m3 per row) into LDS; two LDS stages hold slabs
// kt and kt+1 (section 四: pipeline stages hide the global-memory latency).
//
// Schedule.  A gfx950 workgroup of eight waves places waves w and w+4 on the
// same SIMD, one from each group.  Each group alternates a memory phase
// (read one k-tile's fragments from LDS into registers, issue the direct
// HBM -> LDS copies of a later k-tile) with a compute phase (a whole
// k-tile of MFMAs from registers), and the two groups are half a period
// apart, held there by workgroup barriers: group 0 starts a period with its
// memory phase, group 1 with its compute phase.  So on each SIMD one wave
// multiplies while the other moves data, and no copy instruction sits
// between MFMAs: under load a direct-to-LDS copy holds its wave's in-order
// issue for about a hundred cycles.
//
// LDS holds two A slabs and three B slabs (5 x 32 KiB = the whole 160 KiB):
// B of k-tile kt+2 is copied while k-tiles kt and kt+1 are both still
// live.  Each group waits for its own copies before the barrier that
// precedes their first reader.  After the last barrier group 0 runs its
// epilogue while group 1 still multiplies the last k-tile.
//
// Copies are raw buffer loads straight into LDS.  Copy q of a thread moves
// 16 bytes of slab row r0 + 32q (r0 = thread / 8): the buffer resource starts
// at that block of 32 rows and its record count ends at the operand's last
// real row, so a lane whose row lies past M (or N) reads zeros and touches
// no memory; the per-lane offset (row r0, swizzled chunk) is the same for
// every copy and every k-tile, and the k-tile's byte offset is a scalar.
//
// kBT: B is N-contiguous (a row-major K x N matrix, 16-bit).  Its slab holds
// the k-tile's 64 rows of k, each the tile's 256 columns of n (512 bytes,
// 16-byte chunk c of row r stored at chunk c ^ 4 (r % 4)); copy q moves rows
// 8q .. 8q + 7 (the scalar offset carries the row), and columns past N read
// the last whole chunk of the row (never stored).  A B fragment is two
// ds_read_b64_tr_b16 (quarter-wave lane j receives element e from the
// 8 bytes lane 4 e + j / 4 addresses, at position j % 4), so lane a of a
// quarter-wave addresses row k0 + a / 4, columns n0 + 4 (a % 4) .. and lane
// j gets B[k0 .. k0 + 3][n0 + j].  The swizzle term 4 (r % 4) sits in
// address bits 6-7, which hold nothing else, so the wave's four 32-column
// fragments are one base XOR 64 j.
#include "gemm_common.hpp"

namespace tla {
namespace {

template <int kCode, bool kBT = false, bool kAT = false>
__global__ __launch_bounds__(512) void gemm_pingpong_kernel(const GemmParams p) {
  using Atom = MfmaAtom<kCode>;
  using Frag = typename Atom::Frag;
  constexpr int kRowBytes = 128;
  using Swz = typename Slab<kRowBytes>::Swz;
  constexpr int kChunks = Slab<kRowBytes>::kChunks;
  constexpr int EB = elem_bytes(kCode);
  constexpr int BK = kRowBytes / EB;            // K elements per k-tile
  constexpr int BM = 256, BN = 256;
  constexpr int WM = 64, WN = 128;              // wave tile
  constexpr int FM = WM / 32, FN = WN / 32;     // MFMA tiles per wave
  constexpr int KSTEPS = BK / Atom::kK;         // MFMA k-steps per k-tile
  constexpr int kSub = Atom::kLaneBytes / 16;   // 16-byte reads per fragment
  constexpr int kStepBytes = Atom::kK * EB;
  constexpr int SLAB = BM * kRowBytes;          // 32 KiB: one operand, one k-tile
  constexpr int B_BASE = 2 * SLAB;              // LDS: [A0 A1 | B0 B1 B2]
  constexpr int kCopies = SLAB / (256 * 16);    // 16-byte copies per thread per slab
  static_assert(BK % Atom::kK == 0 && kCopies == 8, "k-tile geometry");
  static_assert((1 << Slab<kRowBytes>::kRowShift) * kChunks <= 32,
                "the swizzle repeats within 32 rows");
  static_assert(5 * SLAB <= 160 * 1024, "LDS budget");
  static_assert(!kBT || EB == 2, "N-contiguous B: 16-bit operands");
  static_assert(!kAT || EB == 2, "M-contiguous A: 16-bit operands");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[5 * SLAB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                    // 0: waves 0-3, 1: waves 4-7
  const int t = tid & 255;                      // thread index inside the group
  int tm, tn;
  schedule(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm0 = 128 * grp + WM * (wave & 1), wn0 = WN * ((wave >> 1) & 1);
  const int KT = (p.K + BK - 1) / BK;
  const int KTf = p.K / BK;  // whole k-tiles; tile KTf, if K ends inside it, is ragged

  // ---- copies: group 0 moves A (two LDS slots), group 1 moves B (three
  // slots), 8 instructions per slab.  Thread t fills slot byte 16 (t + 256q)
  // (lane-linear), i.e. row r0 + 32q, physical chunk t % 8, and fetches the
  // logical chunk the swizzle puts there; rows 32q.. of the tile start the
  // buffer resource of copy q, whose record count ends at the last real row.
  const int r0 = t / kChunks;
  const int64_t rb = (grp == 0 ? p.a_sr : p.b_sr) * EB;   // row pitch in bytes
  const uint8_t* op = (grp == 0 ? p.A + m0 * rb : p.B + n0 * rb);  // the tile's first row
  const int rows_left = (grp == 0 ? p.M - m0 : p.N - n0); // real rows from there on
  uint32_t voff = (uint32_t)(r0 * rb + Swz::chunk(r0, t % kChunks) * 16);
  const int lds_op = grp == 0 ? 0 : B_BASE;
  int recs[kCopies];
  static_for<kCopies>([&](auto q) {
    recs[q] = (int)(min(max(rows_left - 32 * (int)q, 0), 32) * rb);
  });
  // per group: the byte step of a k-tile, and (N-contiguous B) of a copy
  uint32_t kt_bytes = kRowBytes, q_bytes = 0;
  const uint8_t* qbase = op;
  int64_t q_stride = 32 * rb;
  if constexpr (kBT) {
    if (grp == 1) {
      // slab chunk t + 256 q: row r0 = t / 32 (+ 8 q), stored chunk t % 32
      // holding columns n0 + 8 ((t % 32) ^ 4 (r0 % 4)) .. + 7
      const int64_t ldb = p.b_sk;
      const int rt = t >> 5;
      const int n = min(n0 + 8 * ((t & 31) ^ (4 * (rt & 3))), p.N - 8);
      voff = (uint32_t)((rt * ldb + n) * EB);
      kt_bytes = (uint32_t)(BK * ldb * EB);
      q_bytes = (uint32_t)(8 * ldb * EB);
      qbase = p.B;
      q_stride = 0;
      const int64_t whole = (int64_t)p.K * ldb * EB;
      static_for<kCopies>([&](auto q) { recs[q] = (int)min(whole, (int64_t)0x7FFFFFFF); });
    }
  }
  if constexpr (kAT) {
    if (grp == 0) {
      // the same for an M-contiguous A (column-major M x K, pitch lda):
      // row rt (+ 8 q) of k, stored chunk t % 32 holding columns
      // m0 + 8 ((t % 32) ^ 4 (rt % 4)) .. + 7, clamped to the last chunk of M
      const int64_t lda = p.a_sk;
      const int rt = t >> 5;
      const int m = min(m0 + 8 * ((t & 31) ^ (4 * (rt & 3))), p.M - 8);
      voff = (uint32_t)((rt * lda + m) * EB);
      kt_bytes = (uint32_t)(BK * lda * EB);
      q_bytes = (uint32_t)(8 * lda * EB);
      qbase = p.A;
      q_stride = 0;
      const int64_t whole = (int64_t)p.K * lda * EB;
      static_for<kCopies>([&](auto q) { recs[q] = (int)min(whole, (int64_t)0x7FFFFFFF); });
    }
  }
  // The ragged last k-tile (K a multiple of the 16-byte chunk): a lane whose
  // K-contiguous chunk lies past K reads from past every record, so the
  // range check returns zeros; the rows past K of a k-rows slab (an M- or
  // N-contiguous operand) are past its records already.
  uint32_t voff_tail = voff;
  if ((grp == 0 && !kAT) || (grp == 1 && !kBT)) {
    if (Swz::chunk(r0, t % kChunks) * 16 >= (p.K - KTf * BK) * EB) voff_tail = 0x80000000u;
  }
  // Copy q of k-tile kt into `slot`.  A copy past the last k-tile still runs
  // (so the instruction stream and the wait counts never change) but with no
  // records: it writes zeros into a slot nobody reads any more.
  auto copy_one = [&](int kt, int slot, bool live, auto q) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(qbase + (int64_t)q * q_stride), 0, recs[q] & -(int)live, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(smem + lds_op + slot * SLAB + q * 4096 +
                                                     (wave & 3) * 1024),
        16, kt == KTf ? voff_tail : voff, (uint32_t)kt * kt_bytes + (uint32_t)q * q_bytes, 0, 0);
  };
  auto copy_slab = [&](int kt, int slot, bool live) {
    static_for<kCopies>([&](auto q) { copy_one(kt, slot, live, q); });
  };

  // ---- fragments: one base register per k-step; the A slot and the 32-row
  // fragment are immediates, the B slot (three of them: immediates would
  // pass 64 KiB) is added into the B bases as they move from slot to slot.
  // A 32-byte (e4m3) fragment is logical chunks 2u, 2u+1 of the row: the
  // swizzle XORs the chunk index, so the second chunk sits at the first
  // one's address XOR 16 (every other term of the address is a multiple of
  // 128), formed in the loop rather than held.
  static_assert(kSub == 1 || (Atom::kLaneBytes == 32 && kStepBytes % 32 == 0), "chunk pairs");
  uint32_t fa[kAT ? 1 : KSTEPS], fb[kBT ? 1 : KSTEPS];
  static_for<KSTEPS>([&](auto ks) {
    const int c = (ks * kStepBytes + (lane >> 5) * Atom::kLaneBytes) / 16;
    const int ra = wm0 + (lane & 31), rbw = wn0 + (lane & 31);
    if constexpr (!kAT) fa[ks] = (uint32_t)(ra * kRowBytes + Swz::chunk(ra, c) * 16);
    if constexpr (!kBT)
      fb[ks] = (uint32_t)(B_BASE + rbw * kRowBytes + Swz::chunk(rbw, c) * 16);  // B slot 0
  });
  if constexpr (kAT) {
    // as for an N-contiguous B below, with rows m = wm0 + ... of A slot 0
    // (wm0 is a multiple of 64, so fragment i is again XOR 64 i)
    const int qw = lane >> 4, a4 = lane & 15;
    const int k = 8 * (qw >> 1) + (a4 >> 2);
    const int m = wm0 + 16 * (qw & 1) + 4 * (a4 & 3);
    fa[0] = (uint32_t)(k * 512 + (((m >> 3) ^ (4 * (k & 3))) * 16) + (m & 7) * 2);
  }
  if constexpr (kBT) {
    // transpose read h of k-step ks for lane a of quarter-wave qw: row
    // k = 16 ks + 8 (qw / 2) + 4 h + a / 4, columns n = wn0 + 16 (qw % 2) +
    // 4 (a % 4) of the first 32-column fragment, stored chunk
    // (n / 8) ^ 4 (k % 4).  k % 4 = a / 4 whatever ks and h, so one base
    // (ks = h = 0) serves all: + 8192 ks + 2048 h, and XOR 64 j for
    // fragment j
    const int qw = lane >> 4, a4 = lane & 15;
    const int k = 8 * (qw >> 1) + (a4 >> 2);
    const int n = wn0 + 16 * (qw & 1) + 4 * (a4 & 3);
    fb[0] = (uint32_t)(B_BASE + k * 512 + (((n >> 3) ^ (4 * (k & 3))) * 16) + (n & 7) * 2);
  }
  Frag a[KSTEPS][FM], b[KSTEPS][FN];
  auto lds_frag = [&](uint32_t base, int imm) -> Frag {
    if constexpr (kSub == 1) {
      return *(const i32x4*)(smem + base + imm);
    } else {
      uint32_t base_hi = base ^ 16u;
      asm volatile("" : "+v"(base_hi));  // keep the XOR in the loop
      const i32x4 lo = *(const i32x4*)(smem + base + imm);
      const i32x4 hi = *(const i32x4*)(smem + base_hi + imm);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  // k-tile kt: A slot kt % 2 (immediate), B slot kt % 3 (in fb); afterwards
  // fb moves on to B slot (kt + 1) % 3
  auto lds_frag_t = [&](uint32_t addr) -> Frag {
    typedef int s32x2 __attribute__((ext_vector_type(2)));
    const s16x4 lo = ds_read_tr16(smem + addr);
    const s16x4 hi = ds_read_tr16(smem + addr + 2048);
    const s32x2 l2 = __builtin_bit_cast(s32x2, lo), h2 = __builtin_bit_cast(s32x2, hi);
    return Frag{l2[0], l2[1], h2[0], h2[1]};
  };
  auto read_frag = [&](int kt, auto r) {
    constexpr int ks = r / (FM + FN), f = r % (FM + FN);
    if constexpr (f < FM && kAT)
      a[ks][f] = lds_frag_t((fa[0] ^ (64u * f)) + 8192 * ks + (kt & 1) * SLAB);
    else if constexpr (f < FM)
      a[ks][f] = lds_frag(fa[ks], (kt & 1) * SLAB + f * 32 * kRowBytes);
    else if constexpr (kBT)
      b[ks][f - FM] = lds_frag_t((fb[0] ^ (64u * (f - FM))) + 8192 * ks);
    else
      b[ks][f - FM] = lds_frag(fb[ks], (f - FM) * 32 * kRowBytes);
  };
  auto advance_b = [&](int kt) {
    const int step = (kt % 3 == 2) ? -2 * SLAB : SLAB;
    static_for<kBT ? 1 : KSTEPS>([&](auto ks) { fb[ks] += step; });
  };
  // A memory phase: read k-tile kt's fragments and copy k-tile ct into
  // `slot`.  Under load the copy path accepts a direct-to-LDS copy only every
  // few dozen cycles, and a wave issues in order, so the copies go out
  // between the LDS reads (kReads / kCopies fragments after each copy, the
  // remainder spread over the first copies): the TA and the LDS then work
  // side by side instead of one after the other.  Measured per k-tile of
  // 256 x 256 x 128 bytes: 2508 cycles interleaved against 2590 with the
  // copies after the reads (16-bit), 3728 against 3952 (reads first) and
  // 4276 (copies first) for e4m3.
  constexpr int kReads = KSTEPS * (FM + FN);  // fragments per k-tile
  constexpr int kPer = kReads / kCopies, kRem = kReads % kCopies;
  // LDS read instructions of fragments [first, first + n)
  auto read_insts = [](int first, int n) constexpr {
    int c = 0;
    for (int r = first; r < first + n; ++r)
      c += (r % (FM + FN) < FM) ? (kAT ? 2 : kSub) : (kBT ? 2 : kSub);
    return c;
  };
  auto memory_phase = [&](int kt, int ct, int slot, bool live) {
    __builtin_amdgcn_sched_barrier(0);
    static_for<kCopies>([&](auto q) {
      copy_one(ct, slot, live, q);
      constexpr int first = kPer * q + (q < kRem ? q : kRem);
      constexpr int n = kPer + (q < kRem ? 1 : 0);
      static_for<n>([&](auto u) { read_frag(kt, std::integral_constant<int, first + u>{}); });
    });
    static_for<kCopies>([&](auto q) {
      constexpr int first = kPer * q + (q < kRem ? q : kRem);
      constexpr int n = kPer + (q < kRem ? 1 : 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, read_insts(first, n), 0);
    });
    advance_b(kt);
    __builtin_amdgcn_sched_barrier(0);
  };
  f32x16 acc[FM][FN];
  static_for<FM>([&](auto i) { static_for<FN>([&](auto j) { acc[i][j] = f32x16{}; }); });
  // one k-tile of MFMAs, fenced off from the scheduler on both sides so that
  // no wait or memory instruction of a neighbouring phase moves into it
  auto compute = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    static_for<KSTEPS * FM * FN>([&](auto idx) {
      constexpr int ks = idx / (FM * FN), i = (idx / FN) % FM, j = idx % FN;
      Atom::mma(acc[i][j], b[ks][j], a[ks][i]);
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  auto wait_lgkmcnt0 = [&]() { __builtin_amdgcn_s_waitcnt(0xC07F); };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Each group runs its own program with exactly one MFMA sequence; copies
  // are issued only between LDS reads.  Period kt ends at barrier 2kt+1:
  //   group 0: read k-tile kt's fragments and copy A of kt+1 into A slot
  //     (kt+1)%2 (it held kt-1, read by both groups in period kt-1), then
  //     multiply kt and wait for its copies;
  //   group 1: multiply kt-1 (fragments read in period kt-1), then read
  //     kt's fragments and copy B of kt+2 into B slot (kt+2)%3 (it held
  //     kt-1), then wait for B of kt+1 (copied in period kt-1); in period
  //     0 it only reads.
  // Every slab is thus complete one barrier before its first reader.  A
  // second barrier splits each period between its halves: group 0 reads
  // while group 1 multiplies, then the other way round.  An MFMA holds its
  // wave's issue for its whole run, so without the split group 0 starts
  // multiplying before group 1 is done, both share the matrix core and the
  // period grows (16-bit: 3084 cycles per k-tile against 2508; the e4m3
  // 8192^3 GEMM with GELU: 440 us with one barrier per period, 396 us with
  // two).
  //
  // Group 1's second barrier is skipped after the last k-tile, and the
  // compiler is free to sink the MFMAs, plain register arithmetic, past
  // such a conditional barrier into the next period (it does so for e4m3,
  // which then measured 3664 cycles per k-tile): an empty asm reading every
  // accumulator keeps them in front of it.
  if (KT > 0) {
    if (grp == 0) {
      copy_slab(0, 0, true);
      wait_vmcnt<0>();
      barrier();
      for (int kt = 0; kt < KT; ++kt) {
        memory_phase(kt, kt + 1, (kt + 1) & 1, kt + 1 < KT);
        wait_lgkmcnt0();
        barrier();
        compute();
        wait_vmcnt<0>();                             // A of kt+1 landed
        barrier();
      }
    } else {
      copy_slab(0, 0, true);
      copy_slab(1, 1, KT > 1);
      wait_vmcnt<kCopies>();
      barrier();
      barrier();
      // one iteration reads k-tile kt (end of period kt) and multiplies it
      // (start of period kt+1): the fragments never live across iterations
      for (int kt = 0; kt < KT; ++kt) {
        memory_phase(kt, kt + 2, (kt + 2) % 3, kt + 2 < KT);
        wait_lgkmcnt0();
        wait_vmcnt<kCopies>();                       // B of kt+1 landed
        barrier();
        compute();
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) asm volatile("" ::"v"(acc[i][j]));
        if (kt + 1 < KT) barrier();
      }
      wait_vmcnt<0>();  // the last (record-less) copies
    }
  }
  // Every LDS read of the main loop finished before the last barrier and no
  // copy is in flight, so the slots are free for the epilogue: group 0
  // starts while group 1 still multiplies the last k-tile.
  epilogue_tiles<FM, FN>(p, m0 + wm0, n0 + wn0, lane, acc, smem + wave * (32 * FM) * (64 * FN));
}

}  // namespace

int launch_pingpong(const GemmParams& p0, int a_type, hipStream_t stream, bool bt, bool at) {
  GemmParams p = p0;
  int64_t grid;
  set_grid(p, 256, 256, &grid);
  if (grid <= 0) return TLA_OK;
  if (grid > 0x7FFFFFFF) return TLA_ERR_UNSUPPORTED;
  if (at) {
    if (a_type == kBF16 && bt)
      hipLaunchKernelGGL((gemm_pingpong_kernel<kBF16, true, true>), dim3((unsigned)grid),
                         dim3(512), 0, stream, p);
    else if (a_type == kBF16)
      hipLaunchKernelGGL((gemm_pingpong_kernel<kBF16, false, true>), dim3((unsigned)grid),
                         dim3(512), 0, stream, p);
    else if (a_type == kF16 && bt)
      hipLaunchKernelGGL((gemm_pingpong_kernel<kF16, true, true>), dim3((unsigned)grid),
                         dim3(512), 0, stream, p);
    else if (a_type == kF16)
      hipLaunchKernelGGL((gemm_pingpong_kernel<kF16, false, true>), dim3((unsigned)grid),
                         dim3(512), 0, stream, p);
    else
      return TLA_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
  }
  if (bt) {
    if (a_type == kBF16)
      hipLaunchKernelGGL((gemm_pingpong_kernel<kBF16, true>), dim3((unsigned)grid), dim3(512), 0,
                         stream, p);
    else if (a_type == kF16)
      hipLaunchKernelGGL((gemm_pingpong_kernel<kF16, true>), dim3((unsigned)grid), dim3(512), 0,
                         stream, p);
    else
      return TLA_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
  }
  switch (a_type) {
    case kBF16:
      hipLaunchKernelGGL(gemm_pingpong_kernel<kBF16>, dim3((unsigned)grid), dim3(512), 0, stream, p);
      break;
    case kF16:
      hipLaunchKernelGGL(gemm_pingpong_kernel<kF16>, dim3((unsigned)grid), dim3(512), 0, stream, p);
      break;
    case kE4M3:
      hipLaunchKernelGGL(gemm_pingpong_kernel<kE4M3>, dim3((unsigned)grid), dim3(512), 0, stream, p);
      break;
    default:
      return TLA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? TLA_OK : TLA_ERR_HIP;
}

const void* pingpong_kernel(int a_type) {
  switch (a_type) {
    case kBF16: return (const void*)gemm_pingpong_kernel<kBF16>;
    case kF16: return (const void*)gemm_pingpong_kernel<kF16>;
    case kE4M3: return (const void*)gemm_pingpong_kernel<kE4M3>;
    default: return nullptr;
  }
}

}  // namespace tla
