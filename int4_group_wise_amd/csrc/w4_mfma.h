// Matrix-core operand helpers of the decode kernels (v_mfma_f32_16x16x32_bf16
// with 16 weight rows as the B operand): the nibble -> bf16 decode of one code
// word in the slot order pair_x gives the activations, and the 4 x 4 transpose
// of code words across the lane quarters that makes every MFMA sum 32
// contiguous columns.
#pragma once
#include "w4_device.h"
#include "w4_dot.h"

namespace w4 {

// 8 nibbles (column j at bits 4j) -> 8 bf16 values 128 + u in slot order
// (c0, c4, c1, c5, c2, c6, c3, c7), matching pair_x on the activation side.
__device__ __forceinline__ bf16x8_t decode_word(uint32_t d, uint32_t m) {
  const u32x4 v = {and_or(d, m, kMagic), and_or(d >> 4, m, kMagic), and_or(d >> 8, m, kMagic),
                   and_or(d >> 12, m, kMagic)};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Register i of lane quarter q <- register q of lane quarter i (4 x 4
// transpose across the quarters of the wave).
__device__ __forceinline__ void transpose_quarters(uint32_t (&d)[4]) {
  auto r02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
  auto r13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
  auto r01 = __builtin_amdgcn_permlane16_swap(r02[0], r13[0], false, false);
  auto r23 = __builtin_amdgcn_permlane16_swap(r02[1], r13[1], false, false);
  d[0] = r01[0]; d[1] = r01[1]; d[2] = r23[0]; d[3] = r23[1];
}

}  // namespace w4
