// Device-side helpers shared by the libw4 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

constexpr int kWave = 64;

// Plain vector types (HIP's uint4 is a union-based struct whose copies can
// defeat register promotion; these stay in registers).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) double f64x2_t;

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

// Zero-points of one weight row: one per byte ([N, NG]), or packed two per
// byte ([N, ceil(NG/2)], group 2j in the low nibble of byte j, group 2j + 1 in
// the high nibble).
// Branch-free (pk is 0 or 1), so that a zero-point load does not end the
// basic block it sits in and force a wait for the loads issued before it.
// byte(g) and of(byte, g) split the read into the load and the extraction,
// for kernels that issue many loads before using any (as zero_byte/zero_of
// below).
struct ZeroRow {
  const uint8_t* p;
  uint32_t pk;   // 1: packed two per byte
  __device__ __forceinline__ uint32_t byte(int64_t g) const { return p[g >> pk]; }
  __device__ __forceinline__ uint32_t of(uint32_t b, int64_t g) const {
    return (b >> (4u * (static_cast<uint32_t>(g) & pk))) & (0xFFu >> (4u * pk));
  }
  __device__ __forceinline__ uint32_t operator[](int64_t g) const { return of(byte(g), g); }
};
__device__ __forceinline__ ZeroRow zero_row(const uint8_t* z, int64_t n, int64_t NG, int packed) {
  const uint32_t pk = packed ? 1u : 0u;
  return ZeroRow{z ? z + n * ((NG + pk) >> pk) : z, pk};
}

// The same read with the layout fixed at compile time (PK 0: one per byte,
// PK 1: packed two per byte), for kernels instantiated per layout, in two
// steps: zero_byte loads the byte holding group g's zero-point, zero_of takes
// the zero-point out of it.  A kernel that issues many loads before using any
// calls zero_of at the use, so that no arithmetic on a loaded byte sits among
// the loads (it would make the wave wait for every load issued before it).
template <int PK>
__device__ __forceinline__ uint32_t zero_byte(const uint8_t* z, int64_t n, int64_t NG, int64_t g) {
  if constexpr (PK == 0) return z[n * NG + g];
  else return z[n * ((NG + 1) >> 1) + (g >> 1)];
}
template <int PK>
__device__ __forceinline__ uint32_t zero_of(uint32_t byte, uint32_t g) {
  if constexpr (PK == 0) return byte;
  else return (byte >> (4u * (g & 1u))) & 0xFu;
}

// 0x0F0F0F0F in a VGPR, hidden from the compiler.  After `d & 0x0F0F0F0F`
// with the constant it knows every byte's high nibble is zero and extracts
// bytes 1..3 with v_bfe_u32 before converting; with the mask in a register
// each byte converts with one v_cvt_f32_ubyte{0..3}.  Read by VALU ops only.
__device__ __forceinline__ uint32_t byte_nibble_mask() {
  uint32_t r;
  asm volatile("v_mov_b32 %0, 0x0F0F0F0F" : "=v"(r));
  return r;
}

// ---------------------------------------------------------------------------
// Group-wise quantization of one lane's chunk of 8 values (columns 8j ..
// 8j+7); columns past the row end must hold 0 and cnt is the number of valid
// columns (<= 0 for idle lanes, which still take part in the reduction).  The
// group is an aligned block of lpg lanes (a power of two <= 64) of one wave.
// sc, zf receive the group's scale and zero-point (8 for signed codes); the
// result is the packed code word, column 8j + e in nibble e.
//
// Division.  Only rint(fp32(w / s)) is needed.  With r = rcp(s) (relative
// error <= 2^-23) and t = fp32(w r): |w / s| <= 15 (1 + 2^-23), as the group
// statistics come from the same values, hence |t - w / s| < 2^-18.4, and
// fp32(w / s) is within 2^-20 of w / s, so |t - fp32(w / s)| < 2^-18.  When t
// is farther than 2^-16 from the nearest half-integer, rint(t) ==
// rint(fp32(w / s)); otherwise, and whenever r is not finite, the value is
// redone with the IEEE division.  The codes are therefore exactly those of
// the plain division (values are finite).
// ---------------------------------------------------------------------------
constexpr float kTieMargin = 0.5f - 0x1p-16f;

// max over the lanes of an aligned block of `lpg` lanes (a power of two <= 64)
__device__ __forceinline__ float group_max(float m, int lpg) {
  if (lpg > 1) m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
  if (lpg > 2) m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
  if (lpg > 4) m = fmaxf(m, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(m), 0x1F | (4 << 10))));
  if (lpg > 8) m = fmaxf(m, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(m), 0x1F | (8 << 10))));
  if (lpg > 16) m = fmaxf(m, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(m), 0x1F | (16 << 10))));
  if (lpg > 32) m = fmaxf(m, __shfl_xor(m, 32, kWave));
  return m;
}

// group scale and zero-point (8 for signed codes) from the chunks of the
// group's lpg lanes: hi = max(0, max w), nl = max(0, max -w) (signed: max |w|)
// group_max with the group width fixed at compile time (no branches)
template <int LPG>
__device__ __forceinline__ float group_max_t(float m) {
  if constexpr (LPG > 1) m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
  if constexpr (LPG > 2) m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
  if constexpr (LPG > 4) m = fmaxf(m, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(m), 0x1F | (4 << 10))));
  if constexpr (LPG > 8) m = fmaxf(m, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(m), 0x1F | (8 << 10))));
  if constexpr (LPG > 16) m = fmaxf(m, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(m), 0x1F | (16 << 10))));
  if constexpr (LPG > 32) m = fmaxf(m, __shfl_xor(m, 32, kWave));
  return m;
}

// fp32(x / D) for x >= 0 without the IEEE division sequence: q0 = fp32(x r)
// with r = fp32(1 / D), then one residual step q = fp32(q0 + fp32(x - q0 D) r)
// (both fused multiply-adds).  For D = 7 and D = 15 this is the correctly
// rounded quotient for every finite x >= 0, subnormals included (checked over
// all of them): the binary expansion of x / D is periodic, so the quotient
// never lies close enough to a rounding boundary for the single residual step
// to land on the wrong side.  x = +inf is passed through (the residual would
// be NaN).
template <int D>
__device__ __forceinline__ float div_const(float x) {
  static_assert(D == 7 || D == 15, "exactness is established for 7 and 15 only");
  constexpr float r = 1.0f / static_cast<float>(D);
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, static_cast<float>(D), x);
  const float q = __builtin_fmaf(e, r, q0);
  return x < __builtin_inff() ? q : x;
}

// rint(fp32(x / s)) for 0 <= x <= 15 s (1 + 2^-23): the reciprocal estimate
// decides unless the quotient is near a half-integer or rcp(s) is not finite,
// as for the weights
__device__ __forceinline__ float rint_quotient(float x, float s) {
  const float rc = __builtin_amdgcn_rcpf(s);
  const float t = x * rc;
  float q = rintf(t);
  if (!(fabsf(t - q) < kTieMargin) || !(rc < __builtin_inff())) q = rintf(x / s);
  return q;
}

// LPG > 0: the group is LPG lanes wide (compile time); LPG == 0: lpg lanes
template <bool ASYM, int LPG = 0>
__device__ __forceinline__ void group_scale(const float v[8], int lpg, float& sc, float& zf) {
  float m1 = 0.0f, m2 = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (ASYM) {
      m1 = fmaxf(m1, v[e]);
      m2 = fmaxf(m2, -v[e]);
    } else {
      m1 = fmaxf(m1, fabsf(v[e]));
    }
  }
  if constexpr (LPG > 0) {
    m1 = group_max_t<LPG>(m1);
    if constexpr (ASYM) m2 = group_max_t<LPG>(m2);
  } else {
    m1 = group_max(m1, lpg);
    if constexpr (ASYM) m2 = group_max(m2, lpg);
  }
  zf = 8.0f;
  if constexpr (ASYM) {
    sc = div_const<15>(m1 + m2);
    if (sc == 0.0f) sc = 1.0f;
    zf = fminf(fmaxf(rint_quotient(m2, sc), 0.0f), 15.0f);
  } else {
    sc = div_const<7>(m1);
    if (sc == 0.0f) sc = 1.0f;
  }
}

// qf = rint(v * rcp(sc)); true when some quotient lies near a half-integer or
// the reciprocal is not finite (then quant8_redo must run)
__device__ __forceinline__ bool quant8_fast(const float v[8], float sc, float qf[8]) {
  const float rc = __builtin_amdgcn_rcpf(sc);
  float dmax = 0.0f;                         // largest |t - rint(t)| over the chunk
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float t = v[e] * rc;
    qf[e] = rintf(t);
    dmax = fmaxf(dmax, fabsf(t - qf[e]));
  }
  return !(dmax < kTieMargin) || !(rc < __builtin_inff());
}

// redo with the IEEE division the quotients that lie near a half-integer
// (about 1 weight in 300 for bf16 weights), or all of them when the
// reciprocal is not finite (s subnormal); other values are left as they are
__device__ __forceinline__ void quant8_redo(const float v[8], float sc, float qf[8]) {
  const float rc = __builtin_amdgcn_rcpf(sc);
  const bool all = !(rc < __builtin_inff());
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float t = v[e] * rc;
    if (all || !(fabsf(t - qf[e]) < kTieMargin)) qf[e] = rintf(v[e] / sc);
  }
}

// unsigned nibbles as bytes: clamp(q + z, 0, 15) (zero-point), or
// clamp(q, -7, 7) + 8 for signed codes, flipped back below.  The signed clamp
// acts only when the scale is subnormal: amax / 7 then rounds with a large
// relative error (amax = 17 * 2^-149 gives s = 2 * 2^-149 and a quotient 8.5)
template <bool ASYM>
__device__ __forceinline__ uint32_t pack8(const float qf[8], float zf, int cnt) {
  uint32_t ev = 0, od = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = ASYM ? fminf(fmaxf(qf[e] + zf, 0.0f), 15.0f) : fminf(fmaxf(qf[e], -7.0f), 7.0f) + 8.0f;
    if (e & 1) od = __builtin_amdgcn_cvt_pk_u8_f32(x, e >> 1, od);
    else ev = __builtin_amdgcn_cvt_pk_u8_f32(x, e >> 1, ev);
  }
  uint32_t packed = ev | (od << 4);
  if constexpr (!ASYM) packed ^= 0x88888888u;
  if (cnt < 8) packed &= cnt > 0 ? (1u << (4 * cnt)) - 1u : 0u;   // nibbles past the row end stay 0
  return packed;
}

template <bool ASYM>
__device__ __forceinline__ uint32_t quantize_chunk8(const float v[8], int cnt, int lpg, float& sc_out, float& zf_out) {
  float sc, zf, qf[8];
  group_scale<ASYM>(v, lpg, sc, zf);
  if (quant8_fast(v, sc, qf)) quant8_redo(v, sc, qf);
  sc_out = sc;
  zf_out = zf;
  return pack8<ASYM>(qf, zf, cnt);
}

}  // namespace w4
