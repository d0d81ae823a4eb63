// Device-side helpers shared by the libw4 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

constexpr int kWave = 64;

// Plain vector types (HIP's uint4 is a union-based struct whose copies can
// defeat register promotion; these stay in registers).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// bf16 <-> fp32.  bf16 is the upper half of an fp32; rounding to bf16 is to
// the nearest value, ties to the even significand, done on the bit pattern so
// that subnormals are kept (no flush) and the result is exactly reproducible.
__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace w4
