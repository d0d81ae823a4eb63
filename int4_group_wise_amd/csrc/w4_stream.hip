// Decode GEMV, streaming form, for gfx950: y = x Wd^T + b with M = 1
// (keras dense.py diff page: Dense._int4_call, the matmul with the
// dequantized kernel then the bias add; PaddleNLP quantization_linear.py page:
// weight_only_linear with group_size).  The group-wise dequantization
// (u - z) * s of each nibble is folded into the dot product:
// sum_k x_k (u_k - z) s = s * (sum_k x_k (128 + u_k) - (128 + z) sum_k x_k).
#include "w4_device.h"
#include "w4_dot.h"
#include "w4_internal.h"

namespace w4 {
namespace {

// ---------------------------------------------------------------------------
// Decode GEMV, M = 1, streaming form (K a multiple of 2048, contiguous groups
// with G % 32 == 0).  A set of P waves owns R consecutive weight rows; in each
// row the 32-column slices are dealt round-robin: lane l of wave h takes
// slices l + 64 (P j + h), j < S, so that a load instruction reads 1 KB of a
// row contiguously.  Every load of the wave is issued before any arithmetic:
// the activations and the bias first, then row by row the code words, scales
// and zero-points.  Loads retire in order, so the arithmetic of row r waits
// only for row r's data and runs while the later rows are still streaming in;
// only the last row's arithmetic is exposed at the end.  The activations are
// loaded and re-paired once per wave for all R rows.  With P = 2 the two
// waves' row sums meet in LDS and the first wave stores them.
// ---------------------------------------------------------------------------
constexpr int kStreamWG = 4;   // waves per workgroup
template <int R, int S, int P, int ZP>   // ZP: 0 no zero-points, 1 one per byte, 2 two per byte
__global__ __launch_bounds__(kStreamWG * kWave) void gemv_stream_kernel(LinearArgs a) {
  constexpr bool ASYM = ZP != 0;
  static_assert(R >= 1 && R <= 16, "at most four four-row reductions");
  static_assert(P == 1 || P == 2, "one or two waves per row set");
  constexpr int H = (R + 3) / 4;   // four-row reductions
  __shared__ float red[kStreamWG][4 * H];
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = w % P;
  // 32-bit offsets from the arrays' bases (the launcher checks they fit), so
  // that every load takes a uniform base and one 32-bit lane offset
  const uint32_t N1 = static_cast<uint32_t>(a.N - 1);
  const uint32_t set = blockIdx.x * (kStreamWG / P) + static_cast<uint32_t>(w / P);
  const uint32_t row0 = set * R;   // rows past N are clamped: computed, not stored
  const uint32_t rowc = min(row0, N1);
  const uint32_t mask = nibble_mask();
  const uint32_t KB = static_cast<uint32_t>(a.K / 2);
  const uint32_t NG = static_cast<uint32_t>(a.NG);
  auto slice = [&](int j) -> uint32_t { return static_cast<uint32_t>(lane) + 64u * (P * j + h); };

  // activations of the lane's slices, 64 bytes each
  u32x4 xr[S][4];
#pragma unroll
  for (int j = 0; j < S; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xr[j][i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a.x) + 64u * slice(j) + 16 * i);
  // after the reduction lane l holds the sum of row row0 + 4 hh + l / 16
  uint32_t braw[H];
#pragma unroll
  for (int hh = 0; hh < H; ++hh) {
    const uint32_t n = min(row0 + 4u * hh + static_cast<uint32_t>(lane >> 4), N1);
    braw[hh] = a.bias ? a.bias[n] : a.x[0];
  }
  __builtin_amdgcn_sched_barrier(0);

  uint32_t g[S];
#pragma unroll
  for (int j = 0; j < S; ++j) g[j] = (32u * slice(j)) / static_cast<uint32_t>(a.G);
  u32x4 cw[R][S];
  float sc[R][S];
  uint32_t zb[R][S];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t n = min(rowc + r, N1);
#pragma unroll
    for (int j = 0; j < S; ++j)
      cw[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.codes + (n * KB + 16u * slice(j))));
#pragma unroll
    for (int j = 0; j < S; ++j) {
      // scales and zero-points are read once per call too: non-temporal
      sc[r][j] = __builtin_nontemporal_load(
          reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.scales) + 4u * (n * NG + g[j])));
      if constexpr (ZP == 1) zb[r][j] = __builtin_nontemporal_load(a.zeros + (n * NG + g[j]));
      if constexpr (ZP == 2) zb[r][j] = __builtin_nontemporal_load(a.zeros + (n * ((NG + 1u) >> 1) + (g[j] >> 1)));
      if constexpr (ZP == 0) zb[r][j] = 8u;
    }
    __builtin_amdgcn_sched_barrier(0);   // issue order = use order, row by row
  }

  // re-pair the activations to the decode's slot order; their sums per slice
  const uint32_t ones = 0x3F803F80u;   // bf16 pair (1.0, 1.0)
  uint32_t xp[S][4][4];
  float xsum[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    xsum[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t in[4] = {xr[j][i][0], xr[j][i][1], xr[j][i][2], xr[j][i][3]};
      pair_x(in, xp[j][i]);
#pragma unroll
      for (int p = 0; p < 4; ++p) xsum[j] = dot2_bf16(xp[j][i][p], ones, xsum[j]);
    }
  }

  float tot[4 * H];
#pragma unroll
  for (int r = 0; r < 4 * H; ++r) tot[r] = 0.0f;
  const uint32_t flip = ASYM ? 0u : 0x88888888u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = dot8(cw[r][j][i] ^ flip, mask, xp[j][i], acc);
      tot[r] += sc[r][j] * (acc - (128.0f + static_cast<float>(zero_of<ZP == 2>(zb[r][j], g[j]))) * xsum[j]);
    }
  }

  float v[H];
#pragma unroll
  for (int hh = 0; hh < H; ++hh) v[hh] = wave_sum4(tot[4 * hh], tot[4 * hh + 1], tot[4 * hh + 2], tot[4 * hh + 3]);
  if constexpr (P == 2) {
    // the second wave of the set hands its sums to the first, which adds them
    // (fixed order: first wave + second wave)
    if (h == 1 && (lane & 15) == 0) {
#pragma unroll
      for (int hh = 0; hh < H; ++hh) red[w][4 * hh + (lane >> 4)] = v[hh];
    }
    __syncthreads();
    if (h == 1) return;
#pragma unroll
    for (int hh = 0; hh < H; ++hh) v[hh] += red[w + 1][4 * hh + (lane >> 4)];
  }
#pragma unroll
  for (int hh = 0; hh < H; ++hh) {
    const uint32_t n = row0 + 4u * hh + static_cast<uint32_t>(lane >> 4);
    const float bias = a.bias ? bf16_to_f32(braw[hh]) : 0.0f;
    if ((lane & 15) == 0 && 4 * hh + (lane >> 4) < R && n <= N1)
      a.y[n] = static_cast<uint16_t>(f32_to_bf16(v[hh] + bias));
  }
}

constexpr int kStreamP = 2;              // waves per row set
constexpr int64_t kStreamSets = 2048;    // row sets per launch, about

}  // namespace

// Rows per wave of the streaming decode GEMV: about two waves per SIMD
// (2048 waves on 256 CUs) when N allows it.
int stream_rows(int64_t N) {
  const int64_t r = (N + kStreamSets - 1) / kStreamSets;
  return r <= 2 ? 2 : r <= 4 ? 4 : r <= 7 ? 7 : r <= 8 ? 8 : r <= 14 ? 14 : 16;
}

namespace {

template <int R, int S, int ZP>
hipError_t launch_stream3(const LinearArgs& a, hipStream_t s) {
  constexpr int sets_per_wg = kStreamWG / kStreamP;
  const int64_t sets = (a.N + R - 1) / R;
  gemv_stream_kernel<R, S, kStreamP, ZP><<<dim3(static_cast<uint32_t>((sets + sets_per_wg - 1) / sets_per_wg)),
                                             dim3(kStreamWG * kWave), 0, s>>>(a);
  return hipGetLastError();
}

template <int ZP>
hipError_t launch_stream2(const LinearArgs& a, hipStream_t s) {
  constexpr int S = 2 / kStreamP;   // K = 4096: 128 slices per row
  switch (stream_rows(a.N)) {
    case 2: return launch_stream3<2, S, ZP>(a, s);
    case 4: return launch_stream3<4, S, ZP>(a, s);
    case 7: return launch_stream3<7, S, ZP>(a, s);
    case 8: return launch_stream3<8, S, ZP>(a, s);
    case 14: return launch_stream3<14, S, ZP>(a, s);
    default: return launch_stream3<16, S, ZP>(a, s);
  }
}

}  // namespace

hipError_t launch_stream(const LinearArgs& a, hipStream_t s) {
  if (!a.asym) return launch_stream2<0>(a, s);
  return a.zpk ? launch_stream2<2>(a, s) : launch_stream2<1>(a, s);
}

// The streaming decode GEMV: M = 1, K = 4096, contiguous groups with G a
// multiple of 32, and code, scale and zero-point arrays whose byte offsets fit
// in 31 bits.
bool stream_ok(const LinearArgs& a) {
  const int64_t lim = int64_t{1} << 31;
  return a.M == 1 && a.g_idx == nullptr && a.K == 4096 && a.G % 32 == 0 && a.N * (a.K / 2) < lim &&
         a.N * a.NG * 4 < lim;
}

}  // namespace w4
