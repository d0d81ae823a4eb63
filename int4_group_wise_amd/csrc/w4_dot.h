// Dot-product helpers of the GEMV kernels: bf16 pair dot products, the
// re-pairing of activations to the nibble order of a code word, the exact
// nibble-to-bf16 decode (0x4300 | u is the bf16 of 128 + u) and the wave sum
// of four per-lane values.
#pragma once
#include "w4_device.h"

namespace w4 {

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Byte selector for v_perm_b32(hi, lo, sel): result byte i = byte sel_i of the
// 8-byte value {hi:lo} (lo = bytes 0..3).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// x values of 8 consecutive columns c0..c0+7 (4 dwords of bf16 pairs) are
// re-paired to match the nibble pairs (c0, c0+4), (c0+1, c0+5), (c0+2, c0+6),
// (c0+3, c0+7) produced from one code word.
__device__ __forceinline__ void pair_x(const uint32_t a[4], uint32_t xp[4]) {
  xp[0] = perm(a[2], a[0], 0x05040100u);   // (x0, x4)
  xp[1] = perm(a[2], a[0], 0x07060302u);   // (x1, x5)
  xp[2] = perm(a[3], a[1], 0x05040100u);   // (x2, x6)
  xp[3] = perm(a[3], a[1], 0x07060302u);   // (x3, x7)
}

// (a & m) | e.  Written in C so that the compiler sees the definition: its
// result often feeds a matrix-core operand, and only instructions the
// compiler can see get the wait states a VALU write needs before an MFMA
// reads the same register.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t e) {
  return (a & m) | e;
}

// The nibble-pair mask 0x000F000F in a VGPR.  Loaded in asm so that the
// compiler cannot fold it into a constant: with the mask in a register and the
// exponent pattern in an SGPR, (a & m) | e selects one v_and_or_b32 (a VOP3
// op here may read one scalar and no literal).  Its only readers are VALU
// ops, so no matrix-core hazard hides behind the asm.
__device__ __forceinline__ uint32_t nibble_mask() {
  uint32_t r;
  asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(r));
  return r;
}

constexpr uint32_t kMagic = 0x43004300u;   // bf16 pair (128, 128): 0x4300 | u == 128 + u

// sum over 8 columns of x * (128 + u); d holds the 8 nibbles (column j at bits 4j).
__device__ __forceinline__ float dot8(uint32_t d, uint32_t m, const uint32_t xp[4], float acc) {
  acc = dot2_bf16(and_or(d, m, kMagic), xp[0], acc);
  acc = dot2_bf16(and_or(d >> 4, m, kMagic), xp[1], acc);
  acc = dot2_bf16(and_or(d >> 8, m, kMagic), xp[2], acc);
  acc = dot2_bf16(and_or(d >> 12, m, kMagic), xp[3], acc);
  return acc;
}

// Wave sums of four values per lane (one per weight row of the wave), all in
// VALU cross-lane operations: a 32-lane swap pairs rows 0/2 and 1/3 across the
// wave halves, a 16-lane swap leaves the partial sums of row r in lanes
// 16r .. 16r + 15, and four DPP steps (rotate by 8 and 4 within the 16-lane
// row, then the two quad swaps) finish every row.  Lane l returns the total of
// row l / 16.  The order of the additions is fixed.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum4(float t0, float t1, float t2, float t3) {
  const auto a02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(t0), __float_as_uint(t2), false, false);
  const auto a13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(t1), __float_as_uint(t3), false, false);
  const float s02 = __uint_as_float(a02[0]) + __uint_as_float(a02[1]);   // lanes 0-31: row 0, 32-63: row 2
  const float s13 = __uint_as_float(a13[0]) + __uint_as_float(a13[1]);   // lanes 0-31: row 1, 32-63: row 3
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
  float v = __uint_as_float(q[0]) + __uint_as_float(q[1]);               // lanes 16r..16r+15: row r
  v = dpp_add<0x128>(v);   // row_ror:8
  v = dpp_add<0x124>(v);   // row_ror:4
  v = dpp_add<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v = dpp_add<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  return v;
}

}  // namespace w4
