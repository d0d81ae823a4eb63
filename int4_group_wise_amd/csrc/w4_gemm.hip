// Prefill path of the W4A16 linear (M > 16) on gfx950: the weight is first
// dequantized to bf16 (w4_codec.hip, the same rounding as w4_dequantize), then
// this bf16 GEMM  y = x . Wd^T + b  runs on the matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation, one bf16 rounding at the end).
// (keras dense.py diff page, Dense._int4_call: dequantize, cast to the compute
// dtype, matmul, bias.)
//
// Both operands are K-contiguous (x [M, K], Wd [N, K]).  A 256-thread
// workgroup computes a 128 x 128 tile of y as a 2 x 2 grid of waves with
// 64 x 64 each (4 x 4 MFMA tiles of 16 x 16), stepping K by 64 through LDS with
// the next K-step prefetched into registers while the current one is used.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kLdsStride = BK + 8;   // bf16 per LDS row: 144 bytes, rows stay 16-byte aligned
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void gemm_bf16_nt_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wd,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * kLdsStride];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int tiles_n = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / tiles_n) * BM;
  const int n0 = (blockIdx.x % tiles_n) * BN;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // A K-step of either operand is 128 rows x 64 columns = 1024 chunks of
  // 8 bf16 (16 bytes); thread t moves chunks t, t+256, t+512, t+768.
  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      const int r = c >> 3, kc = (c & 7) * 8;
      const int gk = k0 + kc;
      const int gm = m0 + r, gn = n0 + r;
      const uint4 zero = {0u, 0u, 0u, 0u};
      ra[i] = (gm < M && gk < K) ? *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(gm) * K + gk) : zero;
      rb[i] = (gn < N && gk < K) ? *reinterpret_cast<const uint4*>(wd + static_cast<int64_t>(gn) * K + gk) : zero;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      const int r = c >> 3, kc = (c & 7) * 8;
      *reinterpret_cast<uint4*>(&As[r * kLdsStride + kc]) = ra[i];
      *reinterpret_cast<uint4*>(&Bs[r * kLdsStride + kc]) = rb[i];
    }
  };

  const int nk = (K + BK - 1) / BK;
  gload(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      const int kof = kk + 8 * (lane >> 4);
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * 64 + i * 16 + (lane & 15)) * kLdsStride + kof]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[(wn * 64 + j * 16 + (lane & 15)) * kLdsStride + kof]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // 16 x 16 accumulator layout: lane holds rows 4*(lane/16) + t, column lane % 16.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 64 + j * 16 + (lane & 15);
    if (n >= N) continue;
    const float b = bias ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + t;
        if (m < M) y[static_cast<int64_t>(m) * N + n] = static_cast<uint16_t>(f32_to_bf16(acc[i][j][t] + b));
      }
    }
  }
}

// Any K (rows not 16-byte aligned): one thread per output, fp32 accumulation.
__global__ __launch_bounds__(256) void gemm_bf16_nt_simple_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wd,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int64_t M, int64_t N, int64_t K) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= M * N) return;
  const int64_t m = idx / N, n = idx % N;
  float acc = 0.0f;
  for (int64_t k = 0; k < K; ++k) acc += bf16_to_f32(x[m * K + k]) * bf16_to_f32(wd[n * K + k]);
  if (bias) acc += bf16_to_f32(bias[n]);
  y[idx] = static_cast<uint16_t>(f32_to_bf16(acc));
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* wd, const uint16_t* bias,
                            uint16_t* y, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  if (K % 8 == 0 && M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    gemm_bf16_nt_kernel<<<dim3(static_cast<uint32_t>(tiles)), dim3(kThreads), 0, s>>>(
        x, wd, bias, y, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
  } else {
    const int64_t total = M * N;
    gemm_bf16_nt_simple_kernel<<<dim3(static_cast<uint32_t>((total + 255) / 256)), dim3(256), 0, s>>>(
        x, wd, bias, y, M, N, K);
  }
  return hipGetLastError();
}

}  // namespace w4
