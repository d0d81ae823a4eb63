// W4A16 linear kernels for gfx950:  y[m, n] = sum_k x[m, k] * Wd[n, k] + b[n]
// (keras dense.py diff page: Dense._int4_call, matmul with the dequantized
// kernel then the bias add; PaddleNLP quantization_linear.py page:
// weight_only_linear with group_size).
//
// Skinny path (decode, M <= 16), HBM-bound: every weight byte is read once.
//   gemv_dot2   contiguous groups, G % 32 == 0, K % 32 == 0, M <= 4.  Each lane
//               streams 16 bytes (32 columns) of a row per load, turns nibble
//               pairs into bf16 pairs with one and-or against the exponent
//               pattern of 128.0 (bf16 0x4300 | u == 128 + u exactly) and
//               accumulates with v_dot2c_f32_bf16.  Per 32-column group slice
//               the offset is removed once:  sum_k x_k (u_k - z) s =
//               s * (sum_k x_k (128 + u_k) - (128 + z) sum_k x_k).
//               Signed codes use u = c ^ 8, z = 8 (two's complement nibble
//               c - 16 [c >= 8] == (c ^ 8) - 8).
//   gemv_generic  any G, K, g_idx: one wave per row, per-element dequantize
//               to the bf16 weight (as the dense path computes it).
// Prefill path (M > 16) lives in w4_gemm.hip.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {
namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Byte selector for v_perm_b32(hi, lo, sel): result byte i = byte sel_i of the
// 8-byte value {hi:lo} (lo = bytes 0..3).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

constexpr int kGemvWaves = 4;   // waves per workgroup
constexpr int kGemvRows = 4;    // weight rows per wave

// x values of 8 consecutive columns c0..c0+7 (4 dwords of bf16 pairs) are
// re-paired to match the nibble pairs (c0, c0+4), (c0+1, c0+5), (c0+2, c0+6),
// (c0+3, c0+7) produced from one code word.
__device__ __forceinline__ void pair_x(const uint32_t a[4], uint32_t xp[4]) {
  xp[0] = perm(a[2], a[0], 0x05040100u);   // (x0, x4)
  xp[1] = perm(a[2], a[0], 0x07060302u);   // (x1, x5)
  xp[2] = perm(a[3], a[1], 0x05040100u);   // (x2, x6)
  xp[3] = perm(a[3], a[1], 0x07060302u);   // (x3, x7)
}

// sum over 8 columns of x * (128 + u); d holds the 8 nibbles (column j at bits 4j).
__device__ __forceinline__ float dot8(uint32_t d, const uint32_t xp[4], float acc) {
  const uint32_t m = 0x000F000Fu, e = 0x43004300u;
  acc = dot2_bf16((d & m) | e, xp[0], acc);
  acc = dot2_bf16(((d >> 4) & m) | e, xp[1], acc);
  acc = dot2_bf16(((d >> 8) & m) | e, xp[2], acc);
  acc = dot2_bf16(((d >> 12) & m) | e, xp[3], acc);
  return acc;
}

template <int MT, bool ASYM>
__global__ __launch_bounds__(kGemvWaves * kWave) void gemv_dot2_kernel(LinearArgs a) {
  const int lane = lane_id();
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kGemvWaves + (threadIdx.x >> 6);
  const int64_t row0 = wave * kGemvRows;
  if (row0 >= a.N) return;
  const int K = static_cast<int>(a.K);
  const int units = K / 32;                    // 32-column slices per row
  const int64_t KB = a.K / 2;
  const int M = static_cast<int>(a.M);
  const uint32_t ones = 0x3F803F80u;           // bf16 pair (1.0, 1.0)

  float tot[kGemvRows][MT];
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) tot[r][m] = 0.0f;

  for (int u0 = 0; u0 < units; u0 += kWave) {
    const int u = u0 + lane;
    if (u < units) {
      // code words of this lane's 32 columns for every row of the wave
      uint4 cw[kGemvRows];
      float sc[kGemvRows];
      float zo[kGemvRows];
      const int g = (32 * u) / static_cast<int>(a.G);
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r) {
        const int64_t n = min(row0 + r, a.N - 1);   // clamped rows are computed, not stored
        cw[r] = *reinterpret_cast<const uint4*>(a.codes + n * KB + 16 * u);
        sc[r] = a.scales[n * a.NG + g];
        zo[r] = ASYM ? 128.0f + static_cast<float>(a.zeros[n * a.NG + g]) : 136.0f;
      }
      // activations of the same 32 columns
      uint32_t xp[MT][4][4];
      float xs[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int mm = min(m, M - 1);
        const uint4* xr = reinterpret_cast<const uint4*>(a.x + static_cast<int64_t>(mm) * a.K + 32 * u);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 q = xr[i];
          const uint32_t t[4] = {q.x, q.y, q.z, q.w};
          pair_x(t, xp[m][i]);
#pragma unroll
          for (int p = 0; p < 4; ++p) s = dot2_bf16(xp[m][i][p], ones, s);
        }
        xs[m] = s;
      }
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r) {
        uint32_t d[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
        if constexpr (!ASYM) {
#pragma unroll
          for (int i = 0; i < 4; ++i) d[i] ^= 0x88888888u;
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float acc = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc = dot8(d[i], xp[m][i], acc);
          tot[r][m] += sc[r] * (acc - zo[r] * xs[m]);
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < kGemvRows; ++r) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float v = wave_sum(tot[r][m]);
      const int64_t n = row0 + r;
      if (lane == 0 && n < a.N && m < M) {
        const float b = a.bias ? bf16_to_f32(a.bias[n]) : 0.0f;
        a.y[static_cast<int64_t>(m) * a.N + n] = static_cast<uint16_t>(f32_to_bf16(v + b));
      }
    }
  }
}

// Any G, K and g_idx, M <= 16: one wave per weight row.  Each lane handles one
// code byte (two columns) at a time, dequantizes to the bf16 weight and
// accumulates all M activation rows in fp32.
template <bool ASYM, bool GIDX>
__global__ __launch_bounds__(kGemvWaves * kWave) void gemv_generic_kernel(LinearArgs a) {
  const int lane = lane_id();
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kGemvWaves + (threadIdx.x >> 6);
  if (n >= a.N) return;
  const int K = static_cast<int>(a.K);
  const int KB = (K + 1) / 2;
  const int M = static_cast<int>(a.M);
  const int G = static_cast<int>(a.G);
  const uint8_t* crow = a.codes + n * static_cast<int64_t>(KB);
  const float* srow = a.scales + n * a.NG;
  const uint8_t* zrow = ASYM ? a.zeros + n * a.NG : nullptr;
  float acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.0f;
  for (int b = lane; b < KB; b += kWave) {
    const uint32_t byte = crow[b];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 2 * b + h;
      if (k < K) {
        const int g = GIDX ? min(max(a.g_idx[k], 0), static_cast<int>(a.NG) - 1) : k / G;
        const int nib = static_cast<int>((byte >> (4 * h)) & 15u);
        const int val = ASYM ? nib - static_cast<int>(zrow[g]) : (nib ^ 8) - 8;
        const float wd = bf16_to_f32(f32_to_bf16(static_cast<float>(val) * srow[g]));
#pragma unroll
        for (int m = 0; m < 16; ++m)
          if (m < M) acc[m] += bf16_to_f32(a.x[static_cast<int64_t>(m) * a.K + k]) * wd;
      }
    }
  }
  const float bias = a.bias ? bf16_to_f32(a.bias[n]) : 0.0f;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (m < M) {
      const float v = wave_sum(acc[m]);
      if (lane == 0) a.y[static_cast<int64_t>(m) * a.N + n] = static_cast<uint16_t>(f32_to_bf16(v + bias));
    }
  }
}

template <int MT>
hipError_t launch_dot2(const LinearArgs& a, hipStream_t s) {
  const int64_t waves = (a.N + kGemvRows - 1) / kGemvRows;
  const dim3 grid(static_cast<uint32_t>((waves + kGemvWaves - 1) / kGemvWaves));
  const dim3 block(kGemvWaves * kWave);
  if (a.asym)
    gemv_dot2_kernel<MT, true><<<grid, block, 0, s>>>(a);
  else
    gemv_dot2_kernel<MT, false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

bool dot2_ok(const LinearArgs& a) {
  return a.g_idx == nullptr && a.G % 32 == 0 && a.K % 32 == 0 && a.M <= 4;
}

}  // namespace

bool skinny_supported(const LinearArgs& a) { return a.M >= 1 && a.M <= 16; }

hipError_t launch_linear_skinny(const LinearArgs& a, hipStream_t s) {
  if (!skinny_supported(a)) return hipErrorInvalidValue;
  if (dot2_ok(a)) {
    if (a.M == 1) return launch_dot2<1>(a, s);
    if (a.M == 2) return launch_dot2<2>(a, s);
    return launch_dot2<4>(a, s);
  }
  const dim3 grid(static_cast<uint32_t>((a.N + kGemvWaves - 1) / kGemvWaves));
  const dim3 block(kGemvWaves * kWave);
  if (a.asym) {
    if (a.g_idx) gemv_generic_kernel<true, true><<<grid, block, 0, s>>>(a);
    else gemv_generic_kernel<true, false><<<grid, block, 0, s>>>(a);
  } else {
    if (a.g_idx) gemv_generic_kernel<false, true><<<grid, block, 0, s>>>(a);
    else gemv_generic_kernel<false, false><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace w4
