// mfma.hpp -- gfx950 matrix-core atoms and their thread/value layouts.
//
// The role the SM80 MMA atom and its (T32, V8) -> (M16, K16) TV layout play
// in "CUTLASS / CuTe 主线" (hpc.payai.win/cutlass, ldmatrix section, Parts
// 2-4) is taken here by the CDNA4 32x32 MFMA instructions on 64-lane
// wavefronts.  The operand loaders and the epilogue derive every lane's
// coordinates from the layouts below, the way make_tiled_copy_A derives the
// copy partition from the MMA layout on that page.
//
// Operand fragments (one 32-row operand tile, K contiguous):
//   lane l holds row l%32 and the (l/32)-th half of the instruction's K slice:
//   KPL contiguous K elements starting at (l/32)*KPL (KPL = 8 for 16-bit,
//   32 for fp8).  As a TV layout into the column-major index i + 32k:
//   ((32, 2), KPL) : ((1, 32*KPL), 32).
//   A and B fragments use the same lane -> K assignment, so the product sums
//   every k exactly once whatever order the hardware walks K in.
// Accumulator (32 x 32 fp32, 16 values per lane), checked on the device:
//   lane l, value r -> (i, j) = (8*(r/4) + 4*(l/32) + r%4, l%32);
//   as a TV layout into i + 32j: ((32, 2), (4, 4)) : ((32, 4), (1, 8)).
#pragma once

#include <stdint.h>

#include "layout.hpp"

namespace tla {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Element-type codes (the public C header's tla_dtype values).
enum ElemCode { kF16 = 0, kBF16 = 1, kE4M3 = 2, kF32 = 3 };

TLA_HD constexpr int elem_bytes(int code) {
  return code == kE4M3 ? 1 : (code == kF32 ? 4 : 2);
}

// Accumulator TV layout of the 32x32 MFMA family.
TLA_HD constexpr Layout<4, int> mfma32_acc_tv() {
  return Layout<4, int>{{32, 2, 4, 4}, {32, 4, 1, 8}};
}
// (i, j) of lane l, accumulator value r.
TLA_HD constexpr int mfma32_acc_row(int l, int r) {
  return mfma32_acc_tv()(Coord<4, int>{{l % 32, l / 32, r % 4, r / 4}}) % 32;
}
TLA_HD constexpr int mfma32_acc_col(int l, int r) {
  return mfma32_acc_tv()(Coord<4, int>{{l % 32, l / 32, r % 4, r / 4}}) / 32;
}

// One 32x32xK MFMA step for a storage type: the instruction, the K it
// consumes and the bytes each lane contributes per operand.
template <int kCode>
struct MfmaAtom;

template <>
struct MfmaAtom<kBF16> {
  static constexpr int kK = 16;            // K per instruction
  static constexpr int kLaneBytes = 16;    // 8 bf16 per lane per operand
  typedef i32x4 Frag;
  static __device__ __forceinline__ void mma(f32x16& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};

template <>
struct MfmaAtom<kF16> {
  static constexpr int kK = 16;
  static constexpr int kLaneBytes = 16;
  typedef i32x4 Frag;
  static __device__ __forceinline__ void mma(f32x16& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  }
};

// OCP e4m3 x e4m3 through the block-scaled f8f6f4 instruction with unit
// scales (E8M0 exponent 127 = 2^0) and format selectors 0 (= E4M3) for both
// operands; the per-tensor scales are applied to the fp32 accumulator in the
// epilogue.
template <>
struct MfmaAtom<kE4M3> {
  static constexpr int kK = 64;
  static constexpr int kLaneBytes = 32;    // 32 e4m3 per lane per operand
  typedef i32x8 Frag;
  static __device__ __forceinline__ void mma(f32x16& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
  }
};

}  // namespace tla
