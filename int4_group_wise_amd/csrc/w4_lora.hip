// LoRA merge of a packed int4 weight (keras dense.py diff page:
// Dense._get_kernel_with_merged_lora): dequantize, add the low-rank update
// c * (A B)^T in the float domain, quantize again with the same group size,
// mode and group map, and pack.
//
//   merged[n, k] = fp32( fp32(v[n, k] * s[n, gid(k)]) + fp32(c * fp32(AB[n, k])) )
//   AB[n, k]     = sum_j A[k, j] B[j, n], accumulated in fp64 for j = 0 .. r-1
//
// A is [K, r] and B is [r, N] as the layer stores them.  Every product of two
// fp32 values is exact in fp64, so the fp64 fused multiply-adds in rank order
// round exactly like the plain definition; one rounding to fp32 follows.  The
// merge's fp32 multiplies and add are compiled with contraction off, so each
// rounds separately as the definition states.
//
// Layout.  A workgroup of 4 waves takes 512 columns (lane l owns columns
// 8l .. 8l+7 of the block) and a block of rows; A^T for its columns (fp32,
// [r][516]) and B for its rows (fp64, [r][rows]) are staged once in LDS.  A
// wave takes 8 rows at a time: per rank step a lane reads its 8 A values and
// the 8 rows' B values (a broadcast read), the next step's reads already in
// flight, and 64 fp64 FMAs update its 8 x 8 accumulator tile.
//
// Epilogue.  Contiguous power-of-two groups of 8 .. 512 columns lie inside
// the block, so the merged values are quantized in registers (group
// statistics by lane reduction) and written over the outputs; the inputs of a
// row are read before its outputs are written, so the merge may run in place.
// Any other grouping (act-order, other group sizes, per-channel) writes the
// merged fp32 weight to the workspace and the codec's quantizer packs it.

#include "w4_device.h"
#include "w4_internal.h"

#include <algorithm>

namespace w4 {
namespace {

constexpr int kLThreads = 256;
constexpr int kLWaves = kLThreads / kWave;
constexpr int kLCols = 8 * kWave;         // columns per workgroup
constexpr int kLStride = kLCols + 4;      // LDS row of A^T (floats): 16-byte aligned, rows on different banks
constexpr int kLRows = 8;                 // rows per wave step
constexpr size_t kLLdsCap = 160 * 1024;   // LDS of one compute unit
constexpr int64_t kLComputeUnits = 256;   // MI355X

// LDS a workgroup may use: the device's per-block limit, at most one CU's LDS
// (the rank-64 A^T tile plus one 32-row B block needs 148 KB)
size_t lora_lds_limit() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
    return 0;
  return std::min(kLLdsCap, static_cast<size_t>(v));
}

__device__ __forceinline__ uint32_t load_code_word(const uint8_t* __restrict__ codes, int64_t off, int cnt,
                                                   bool aligned) {
  if (aligned && cnt >= 8) return *reinterpret_cast<const uint32_t*>(codes + off);
  uint32_t w = 0;
  const int nbytes = min(4, (cnt + 1) / 2);
  for (int b = 0; b < nbytes; ++b) w |= static_cast<uint32_t>(codes[off + b]) << (8 * b);
  return w;
}

// fp32(fp32(v * s) + fp32(c * fp32(ab))): three separately rounded operations
__device__ __forceinline__ float merge_value(int v, float s, float c, double ab) {
#pragma clang fp contract(off)
  const float wd = static_cast<float>(v) * s;
  const float delta = c * static_cast<float>(ab);
  return wd + delta;
}

// QUANT: LPG = G / 8 lanes per group (1 .. 64); otherwise LPG is unused
template <bool ASYM, bool GIDX, bool QUANT, int LPG>
__global__ __launch_bounds__(kLThreads) void lora_merge_kernel(LoraArgs a, int rows_per_block) {
  extern __shared__ __attribute__((aligned(16))) float at[];   // [r][kLStride], then bt
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = static_cast<int>(a.K);
  const int r = a.r;
  const int kb0 = blockIdx.x * kLCols;
  const int64_t n_begin = static_cast<int64_t>(blockIdx.y) * rows_per_block;
  const int64_t n_end = min(a.N, n_begin + rows_per_block);
  double* bt = reinterpret_cast<double*>(at + r * kLStride);   // [r][rows_per_block]

  // B of the block's rows as fp64 (rows past N read as 0); the staging loops
  // are unrolled so that several global loads are in flight per thread
#pragma unroll 8
  for (int i = threadIdx.x; i < r * rows_per_block; i += kLThreads) {
    const int j = i / rows_per_block, q = i - j * rows_per_block;
    const int64_t n = n_begin + q;
    bt[i] = n < a.N ? static_cast<double>(a.b[static_cast<int64_t>(j) * a.N + n]) : 0.0;
  }

  // A^T of the block's columns (columns past K read as 0)
#pragma unroll
  for (int kk = threadIdx.x; kk < kLCols; kk += kLThreads) {
    const int k = kb0 + kk;
    if (k < K) {
      const float* src = a.a + static_cast<int64_t>(k) * r;
      if ((r & 3) == 0) {
#pragma unroll 8
        for (int j = 0; j < r; j += 4) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src + j);
#pragma unroll
          for (int i = 0; i < 4; ++i) at[(j + i) * kLStride + kk] = v[i];
        }
      } else {
#pragma unroll 8
        for (int j = 0; j < r; ++j) at[j * kLStride + kk] = src[j];
      }
    } else {
      for (int j = 0; j < r; ++j) at[j * kLStride + kk] = 0.0f;
    }
  }
  __syncthreads();

  const int k0 = kb0 + 8 * lane;
  const int cnt = K - k0;                              // valid columns of the lane (>= 8: all)
  const int kc = min(k0, K - 1);
  const int64_t KB = (a.K + 1) / 2;
  const bool aligned = (KB & 3) == 0;
  const int NG = static_cast<int>(a.NG);
  const int gl = GIDX ? 0 : kc / static_cast<int>(a.G);   // the lane's group (contiguous groups)
  int ge[8];                                           // group of each column (act-order)
  if constexpr (GIDX) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ge[e] = min(max(a.g_idx[min(kc + e, K - 1)], 0), NG - 1);
  }
  constexpr int lpg = QUANT ? LPG : 1;
  const float c = a.c;

  for (int64_t nb = n_begin + kLRows * w; nb < n_end; nb += kLRows * kLWaves) {
    // the rows' codes and (contiguous groups) scales / zero-points, issued
    // before the rank loop so that their latency hides behind it
    uint32_t cw[kLRows];
    float sc[kLRows];
    int zp[kLRows];
#pragma unroll
    for (int q = 0; q < kLRows; ++q) {
      const int64_t n = min(nb + q, n_end - 1);
      cw[q] = cnt > 0 ? load_code_word(a.codes, n * KB + k0 / 2, cnt, aligned) : 0u;
      if constexpr (!GIDX) {
        sc[q] = a.scales[n * a.NG + gl];
        zp[q] = ASYM ? static_cast<int>(a.zeros[n * a.NG + gl]) : 8;
      }
    }

    double acc[kLRows][8];
#pragma unroll
    for (int q = 0; q < kLRows; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[q][e] = 0.0;
    // rank loop; the reads of step j + 1 are issued before the FMAs of step j
    const float* ap = &at[8 * lane];
    const double* bp = bt + (nb - n_begin);
    f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(ap);
    f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(ap + 4);
    f64x2_t b01 = *reinterpret_cast<const f64x2_t*>(bp);
    f64x2_t b23 = *reinterpret_cast<const f64x2_t*>(bp + 2);
    f64x2_t b45 = *reinterpret_cast<const f64x2_t*>(bp + 4);
    f64x2_t b67 = *reinterpret_cast<const f64x2_t*>(bp + 6);
    for (int j = 0; j < r; ++j) {
      const f32x4_t ca0 = a0, ca1 = a1;
      const double bv[8] = {b01[0], b01[1], b23[0], b23[1], b45[0], b45[1], b67[0], b67[1]};
      const int jn = min(j + 1, r - 1);
      a0 = *reinterpret_cast<const f32x4_t*>(ap + jn * kLStride);
      a1 = *reinterpret_cast<const f32x4_t*>(ap + jn * kLStride + 4);
      b01 = *reinterpret_cast<const f64x2_t*>(bp + jn * rows_per_block);
      b23 = *reinterpret_cast<const f64x2_t*>(bp + jn * rows_per_block + 2);
      b45 = *reinterpret_cast<const f64x2_t*>(bp + jn * rows_per_block + 4);
      b67 = *reinterpret_cast<const f64x2_t*>(bp + jn * rows_per_block + 6);
      __builtin_amdgcn_sched_barrier(0);   // keep the next step's reads ahead of this step's FMAs
      double av[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = static_cast<double>(ca0[i]);
        av[4 + i] = static_cast<double>(ca1[i]);
      }
#pragma unroll
      for (int q = 0; q < kLRows; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[q][e] = __builtin_fma(av[e], bv[q], acc[q][e]);
    }

    // merged values of the 8 rows (a row past the block end repeats the last
    // row's loads and is never stored)
    float m[kLRows][8];
#pragma unroll
    for (int q = 0; q < kLRows; ++q) {
      const int64_t n = min(nb + q, n_end - 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int nib = static_cast<int>((cw[q] >> (4 * e)) & 15u);
        float s;
        int z;
        if constexpr (GIDX) {
          s = a.scales[n * a.NG + ge[e]];
          z = ASYM ? static_cast<int>(a.zeros[n * a.NG + ge[e]]) : 8;
        } else {
          s = sc[q];
          z = zp[q];
        }
        const int v = ASYM ? nib - z : ((nib ^ 8) - 8);
        m[q][e] = merge_value(v, s, c, acc[q][e]);
      }
      if (cnt < 8) {                                   // row tail and idle lanes hold zeros
#pragma unroll
        for (int e = 0; e < 8; ++e) m[q][e] = e < cnt ? m[q][e] : 0.0f;
      }
    }
    if constexpr (QUANT) {
      // each step over all 8 rows, branch-free, so that the rows' reduction
      // and division chains overlap; the rare near-tie redo is one branch
      float gs[kLRows], gz[kLRows], qf[kLRows][8];
#pragma unroll
      for (int q = 0; q < kLRows; ++q) group_scale<ASYM, LPG>(m[q], lpg, gs[q], gz[q]);
      bool redo = false;
#pragma unroll
      for (int q = 0; q < kLRows; ++q) redo |= quant8_fast(m[q], gs[q], qf[q]);
      if (redo) {
#pragma unroll
        for (int q = 0; q < kLRows; ++q) quant8_redo(m[q], gs[q], qf[q]);
      }
#pragma unroll
      for (int q = 0; q < kLRows; ++q) {
        const int64_t n = nb + q;
        if (n >= n_end) break;                         // uniform: rows are per wave
        const uint32_t packed = pack8<ASYM>(qf[q], gz[q], cnt);
        if (cnt > 0) {
          const int64_t off = n * KB + k0 / 2;
          if (aligned && cnt >= 8) {
            *reinterpret_cast<uint32_t*>(a.codes_out + off) = packed;
          } else {
            const int nbytes = min(4, (cnt + 1) / 2);
            for (int b = 0; b < nbytes; ++b) a.codes_out[off + b] = static_cast<uint8_t>(packed >> (8 * b));
          }
          if ((lane & (lpg - 1)) == 0) {
            a.scales_out[n * a.NG + gl] = gs[q];
            if constexpr (ASYM) a.zeros_out[n * a.NG + gl] = static_cast<uint8_t>(gz[q]);
          }
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < kLRows; ++q) {
        const int64_t n = nb + q;
        if (n >= n_end) break;
        if (cnt > 0) {
          float* dst = a.merged + n * a.K + k0;
          if (cnt >= 8 && (a.K & 3) == 0) {
            reinterpret_cast<f32x4_t*>(dst)[0] = f32x4_t{m[q][0], m[q][1], m[q][2], m[q][3]};
            reinterpret_cast<f32x4_t*>(dst)[1] = f32x4_t{m[q][4], m[q][5], m[q][6], m[q][7]};
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e < cnt) dst[e] = m[q][e];
          }
        }
      }
    }
  }
}

template <bool ASYM, bool GIDX, bool QUANT, int LPG>
hipError_t launch_lora3(const LoraArgs& a, hipStream_t s) {
  const size_t lds_max = lora_lds_limit();
  {   // the tiles may pass 64 KB
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = ensure_lds_attribute(reinterpret_cast<const void*>(lora_merge_kernel<ASYM, GIDX, QUANT, LPG>),
                             static_cast<int>(lds_max), dev);
    if (e != hipSuccess) return e;
  }
  // Row blocks: a multiple of the workgroup's 32-row step, small enough that
  // A^T and B fit in LDS, and sized so that the workgroups fill whole rounds
  // of the chip's slots (2 per CU by registers, fewer when LDS is the limit).
  const int64_t cb = (a.K + kLCols - 1) / kLCols;
  const int64_t step = kLRows * kLWaves;
  const size_t a_bytes = static_cast<size_t>(a.r) * kLStride * sizeof(float);
  if (lds_max < a_bytes + static_cast<size_t>(a.r) * step * sizeof(double)) return hipErrorInvalidConfiguration;
  const int64_t rows_fit = static_cast<int64_t>((lds_max - a_bytes) / (static_cast<size_t>(a.r) * sizeof(double)));
  const int64_t cap = std::max<int64_t>(step, rows_fit / step * step);
  int64_t rows = step;
  {
    const size_t lds_step = a_bytes + static_cast<size_t>(a.r) * step * sizeof(double);
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(2, static_cast<int64_t>(kLLdsCap / lds_step)));
    const int64_t slots = kLComputeUnits * per_cu;
    const int64_t rounds = std::max<int64_t>(1, (a.N * cb + slots * cap - 1) / (slots * cap));
    rows = (a.N * cb + slots * rounds - 1) / (slots * rounds);   // rows per workgroup for whole rounds
    rows = std::min(cap, std::max<int64_t>(step, (rows + step - 1) / step * step));
  }
  const size_t lds = a_bytes + static_cast<size_t>(a.r) * rows * sizeof(double);
  const dim3 grid(static_cast<uint32_t>(cb), static_cast<uint32_t>((a.N + rows - 1) / rows));
  lora_merge_kernel<ASYM, GIDX, QUANT, LPG><<<grid, dim3(kLThreads), lds, s>>>(a, static_cast<int>(rows));
  return hipGetLastError();
}

template <bool ASYM>
hipError_t launch_fused(const LoraArgs& a, hipStream_t s) {
  switch (a.G) {
    case 8: return launch_lora3<ASYM, false, true, 1>(a, s);
    case 16: return launch_lora3<ASYM, false, true, 2>(a, s);
    case 32: return launch_lora3<ASYM, false, true, 4>(a, s);
    case 64: return launch_lora3<ASYM, false, true, 8>(a, s);
    case 128: return launch_lora3<ASYM, false, true, 16>(a, s);
    case 256: return launch_lora3<ASYM, false, true, 32>(a, s);
    default: return launch_lora3<ASYM, false, true, 64>(a, s);
  }
}

}  // namespace

bool lora_fused(int64_t K, int64_t G, bool has_g_idx, int64_t r) {
  (void)K;
  return !has_g_idx && G >= 8 && G <= 512 && (G & (G - 1)) == 0 && r <= kLoraMaxRank;
}

size_t lora_workspace_bytes(int64_t N, int64_t K, int64_t G, bool has_g_idx, int64_t r) {
  if (lora_fused(K, G, has_g_idx, r)) return 0;
  return static_cast<size_t>(N) * static_cast<size_t>(K) * sizeof(float);
}

hipError_t launch_lora_merge(const LoraArgs& a, hipStream_t s) {
  if (lora_fused(a.K, a.G, a.g_idx != nullptr, a.r))
    return a.asym ? launch_fused<true>(a, s) : launch_fused<false>(a, s);
  hipError_t e;
  if (a.asym) e = a.g_idx ? launch_lora3<true, true, false, 0>(a, s) : launch_lora3<true, false, false, 0>(a, s);
  else e = a.g_idx ? launch_lora3<false, true, false, 0>(a, s) : launch_lora3<false, false, false, 0>(a, s);
  if (e != hipSuccess) return e;
  const QuantArgs q{a.merged, 0, a.N, a.K, a.G, a.NG, a.asym, a.g_idx, a.codes_out, a.scales_out, a.zeros_out};
  return launch_quantize_pack(q, s);
}

}  // namespace w4
