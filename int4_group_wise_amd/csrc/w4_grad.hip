// Input gradient of the W4A16 linear: dx[m, k] = sum_n dy[m, n] * Wd[n, k]
// (keras dense.py diff page: the custom gradient of the sub-channel int4
// matmul; PaddleNLP quantization_linear.py page: QuantizationLinearFunc
// backward).
//
// M <= 16: the reduction runs over the rows of W, so the N rows are split
// into P slices.  A workgroup of 4 waves (8 for one dy row and 32 columns per
// lane) takes 64 * CPT columns of dx and one slice; a lane owns CPT consecutive columns (32, one 16-byte code load per
// row, when groups are contiguous and a multiple of 32 wide and M <= 4; else
// 8, one dword), streams the code words of its wave's rows (coalesced across
// the wave) and accumulates dy[m, n] * w[n, k] in fp32, the dy values being
// uniform loads.  Each slice writes its fp32 partial [M, K] to the workspace
// and a second kernel adds the P partials in a fixed order (the result does
// not depend on scheduling).  The group size is a multiple of 8, so an
// 8-column piece lies in one group.
//
// M > 16: the weight is dequantized transposed, Wd^T [K, N] bf16, into the
// workspace, and the bf16 GEMM computes dx = dy . (Wd^T)^T.

#include "w4_device.h"
#include "w4_internal.h"

#include <algorithm>

namespace w4 {
namespace {

constexpr int kGThreads = 256;
constexpr int kGWaves = kGThreads / kWave;
// rows of a wave whose loads are issued together: 16 for contiguous groups
// when a lane's accumulators are few (MT * CPT <= 32) and the workgroup has 4
// waves, else 8
template <int MT, int CPT, bool GIDX, int WV>
constexpr int grad_unroll() { return !GIDX && MT * CPT <= 32 && WV == 4 ? 16 : 8; }

// Waves per split workgroup: 8 for one dy row and 32 columns per lane (twice
// the waves per SIMD for the same slices, so that one wave's arithmetic runs
// while another waits for its loads), else 4.
template <int MT, int CPT>
constexpr int grad_waves() { return MT == 1 && CPT == 32 ? 8 : 4; }

// Columns per lane: 32 (one 16-byte code load per row) for contiguous groups
// of a multiple of 32 columns and at most 4 dy rows, else 8 (one dword).
template <int MT, bool WIDE>
constexpr int grad_cpt() { return WIDE && MT <= 4 ? 32 : 8; }

// dy[i] for a wave-uniform index i, read through the scalar cache as the
// aligned dword that holds it (that dword never crosses a page boundary the
// element itself does not, so it stays inside mapped memory)
__device__ __forceinline__ uint32_t load_bf16_uniform(const uint16_t* p, int64_t i) {
  // offsets from the original pointer keep the access in the global address space
  const uint8_t* pb = reinterpret_cast<const uint8_t*>(p);
  const int64_t mis = static_cast<int64_t>(reinterpret_cast<uintptr_t>(pb) & 3);
  const int64_t off = mis + 2 * i;                     // byte offset from the aligned base
  const uint32_t word = *reinterpret_cast<const uint32_t*>(pb - mis + (off & ~static_cast<int64_t>(3)));
  return (off & 2) ? (word >> 16) : (word & 0xFFFFu);
}

// The waves' sums meet in LDS in one step (every wave's buffer at once: 32 KB
// for 4 waves of 32 values per lane, 64 KB for 8) when a lane holds at most 32
// values, else one buffer at a time.
template <int MT, int CPT, int WV>
constexpr bool grad_parallel_sum() { return MT * CPT * kWave * 4 <= 8192 && CPT % (4 * WV) == 0; }

// One workgroup: 64 * CPT columns of dx (lane l owns columns CPT l ..), one
// slice of rows of W; wave w of WV takes rows w, w + WV, ... of the slice.
// The waves' sums are added through LDS in wave order and written as the
// slice's partial (by all waves, an equal share of the columns each, when the
// buffers fit; else by wave 0).
template <bool ASYM, bool GIDX, int MT, int CPT, int WV>
__global__ __launch_bounds__(WV * kWave) void grad_split_kernel(GradArgs a, int rows_per) {
  extern __shared__ __attribute__((aligned(16))) float gsm[];
  constexpr int kW = CPT / 8;                         // code dwords per row
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = static_cast<int>(a.K);
  const int k0 = blockIdx.x * (kWave * CPT) + CPT * lane;
  const int M = static_cast<int>(a.M);
  const int64_t nb = static_cast<int64_t>(blockIdx.y) * rows_per;
  const int64_t ne = min(a.N, nb + rows_per);
  const bool live = k0 < K;
  const int cnt = live ? min(CPT, K - k0) : 0;
  const int64_t KB = (a.K + 1) / 2;
  const int NG = static_cast<int>(a.NG);
  const int kc = min(k0, K - 1);

  // group of the lane's columns (contiguous: one, the chunk lies in one
  // group) or of each of its 8 columns (act-order)
  constexpr int kNGrp = GIDX ? 8 : 1;
  int g[kNGrp];
#pragma unroll
  for (int e = 0; e < kNGrp; ++e)
    g[e] = GIDX ? min(max(a.g_idx[min(kc + e, K - 1)], 0), NG - 1) : kc / static_cast<int>(a.G);
  const bool aligned = cnt == CPT && (KB & 3) == 0;
  const uint32_t bmask = byte_nibble_mask();

  float acc[MT][CPT];
  float corr[MT];                                     // sum over rows of c z (contiguous groups)
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    corr[m] = 0.0f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) acc[m][e] = 0.0f;
  }

  constexpr int kGUnroll = grad_unroll<MT, CPT, GIDX, WV>();
  for (int64_t n0 = nb + w; n0 < ne; n0 += kGUnroll * WV) {
    uint32_t d[kGUnroll][kW];
    float s[kGUnroll][kNGrp];
    uint32_t zb[kGUnroll][kNGrp];   // raw zero-point bytes; the zero-points are taken out at their use
    uint32_t dyr[kGUnroll][MT];   // raw bf16 dy of the block's rows
    // loads of this wave's next kGUnroll rows first (past the slice: reload the last)
#pragma unroll
    for (int u = 0; u < kGUnroll; ++u) {
      const int64_t n = min(n0 + u * WV, ne - 1);
      const uint8_t* crow = a.codes + n * KB + CPT / 2 * (k0 / CPT);
      if (aligned) {
        if constexpr (kW == 4) {
          const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow));
#pragma unroll
          for (int i = 0; i < 4; ++i) d[u][i] = q[i];
        } else {
          d[u][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(crow));
        }
      } else {
        const int nbytes = (cnt + 1) / 2;
#pragma unroll
        for (int i = 0; i < kW; ++i) d[u][i] = 0;
#pragma unroll
        for (int b = 0; b < 4 * kW; ++b)       // static indices: the words stay in registers
          if (b < nbytes) d[u][b >> 2] |= static_cast<uint32_t>(crow[b]) << (8 * (b & 3));
      }
#pragma unroll
      for (int e = 0; e < kNGrp; ++e) {
        s[u][e] = a.scales[n * NG + g[e]];
        zb[u][e] = ASYM ? zero_row(a.zeros, n, NG, a.zpk).byte(g[e]) : 8u;
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) dyr[u][m] = load_bf16_uniform(a.dy, static_cast<int64_t>(min(m, M - 1)) * a.N + n);
    }
#pragma unroll
    for (int u = 0; u < kGUnroll; ++u) {
      // rows past the slice (their loads repeated the last row) are skipped,
      // a uniform branch; rows m >= M (reading row M - 1) add nothing: their
      // dy factor is 0
      const int64_t n = n0 + u * WV;
      if (n >= ne) break;
      float z[kNGrp];
#pragma unroll
      for (int e = 0; e < kNGrp; ++e)
        z[e] = ASYM ? static_cast<float>(zero_row(a.zeros, 0, NG, a.zpk).of(zb[u][e], g[e])) : 8.0f;
      float dm[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float dv = bf16_to_f32(dyr[u][m]);
        dm[m] = m < M ? dv : 0.0f;
      }
      if constexpr (GIDX) {
#pragma unroll
        for (int i = 0; i < kW; ++i) {
          const uint32_t dd = ASYM ? d[u][i] : (d[u][i] ^ 0x88888888u);   // signed q -> q + 8
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float wv = (static_cast<float>((dd >> (4 * e)) & 15u) - z[e]) * s[u][e];
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m][8 * i + e] = __builtin_fmaf(dm[m], wv, acc[m][8 * i + e]);
          }
        }
      } else {
        // one group for the lane's columns: sum c u with c = dy s per row and
        // take sum c z off at the end; the nibbles go to float as unpacked bytes
        float cm[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          cm[m] = dm[m] * s[u][0];
          corr[m] = __builtin_fmaf(cm[m], z[0], corr[m]);
        }
#pragma unroll
        for (int i = 0; i < kW; ++i) {
          const uint32_t dd = ASYM ? d[u][i] : (d[u][i] ^ 0x88888888u);   // signed q -> q + 8
          const uint32_t lo = dd & bmask, hi = (dd >> 4) & bmask;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const float qe = static_cast<float>((lo >> (8 * b)) & 0xFFu);     // column 8i + 2b
            const float qo = static_cast<float>((hi >> (8 * b)) & 0xFFu);     // column 8i + 2b + 1
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              acc[m][8 * i + 2 * b] = __builtin_fmaf(cm[m], qe, acc[m][8 * i + 2 * b]);
              acc[m][8 * i + 2 * b + 1] = __builtin_fmaf(cm[m], qo, acc[m][8 * i + 2 * b + 1]);
            }
          }
        }
      }
    }
  }
  if constexpr (!GIDX) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int e = 0; e < CPT; ++e) acc[m][e] -= corr[m];
  }

  // add the waves' sums in wave order 0, 1, .. (the same order either way)
  float* part = a.partial + static_cast<int64_t>(blockIdx.y) * M * a.K;
  if constexpr (grad_parallel_sum<MT, CPT, WV>()) {
    // every wave stores its sums (register order [m][e], lane-major so the
    // accesses are unit-stride), then wave w adds columns e of its share
    // over the waves and writes them
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int e = 0; e < CPT; ++e) gsm[((w * MT + m) * CPT + e) * kWave + lane] = acc[m][e];
    __syncthreads();
    if (!live) return;
    constexpr int kQ = CPT / WV;                      // columns per wave
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) continue;
      float t[kQ];
#pragma unroll
      for (int i = 0; i < kQ; ++i) {
        const int e = w * kQ + i;
        t[i] = gsm[((0 * MT + m) * CPT + e) * kWave + lane];
#pragma unroll
        for (int src = 1; src < WV; ++src) t[i] += gsm[((src * MT + m) * CPT + e) * kWave + lane];
      }
      float* dst = part + static_cast<int64_t>(m) * a.K + k0 + w * kQ;
      if (cnt == CPT && (a.K & 3) == 0) {
#pragma unroll
        for (int q = 0; q < kQ / 4; ++q) reinterpret_cast<f32x4_t*>(dst)[q] = f32x4_t{t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
      } else {
#pragma unroll
        for (int i = 0; i < kQ; ++i)
          if (w * kQ + i < cnt) dst[i] = t[i];
      }
    }
    return;
  }
  // larger tiles: waves 1..3 in turn through one buffer
  for (int src = 1; src < WV; ++src) {
    if (w == src) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int e = 0; e < CPT; ++e) gsm[(m * CPT + e) * kWave + lane] = acc[m][e];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int e = 0; e < CPT; ++e) acc[m][e] += gsm[(m * CPT + e) * kWave + lane];
    }
    __syncthreads();
  }
  if (w != 0 || !live) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= M) continue;
    float* dst = part + static_cast<int64_t>(m) * a.K + k0;
    if (cnt == CPT && (a.K & 3) == 0) {
#pragma unroll
      for (int q = 0; q < CPT / 4; ++q)
        reinterpret_cast<f32x4_t*>(dst)[q] = f32x4_t{acc[m][4 * q], acc[m][4 * q + 1], acc[m][4 * q + 2], acc[m][4 * q + 3]};
    } else {
#pragma unroll
      for (int e = 0; e < CPT; ++e)
        if (e < cnt) dst[e] = acc[m][e];
    }
  }
}

// dx[i] = bf16(sum over slices p = 0 .. P-1 of partial[p][i]), i over M * K.
// A workgroup takes 64 outputs; its 8 waves sum 8 fixed ranges of slices
// (16 loads in flight per lane: one round when P <= 128), then wave 0 adds
// the 8 range sums in order, so the result does not depend on scheduling.
// At the decode layer's shape (128 slices) 8 ranges of 16 took 12.7-12.8 us
// per gradient call against 13.3 with 16 ranges of 8 (4 of 32: 12.8).
constexpr int kRParts = 8;
constexpr int kRLoads = 16;
__global__ __launch_bounds__(kRParts * kWave) void grad_reduce_kernel(const float* __restrict__ partial,
                                                                      int P, int64_t total, uint16_t* __restrict__ dx) {
  __shared__ float red[kRParts][kWave];
  const int lane = lane_id();
  const int part = threadIdx.x >> 6;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kWave + lane;
  const int64_t ic = min(i, total - 1);
  const int per = (P + kRParts - 1) / kRParts;
  const int p0 = part * per, p1 = min(P, p0 + per);
  float sum = 0.0f;
  for (int p = p0; p < p1; p += kRLoads) {
    float v[kRLoads];
#pragma unroll
    for (int u = 0; u < kRLoads; ++u) v[u] = partial[static_cast<int64_t>(min(p + u, p1 - 1)) * total + ic];
#pragma unroll
    for (int u = 0; u < kRLoads; ++u)
      if (p + u < p1) sum += v[u];
  }
  red[part][lane] = sum;
  __syncthreads();
  if (part != 0 || i >= total) return;
  float t = 0.0f;
#pragma unroll
  for (int q = 0; q < kRParts; ++q) t += red[q][lane];
  dx[i] = static_cast<uint16_t>(f32_to_bf16(t));
}

// Transposed dequantize: wt[k][n] = bf16(value(n, k) * s[n, gid(k)]), a
// 64 x 64 tile per workgroup.  The tile's scale / zero-point rows and group
// indices are staged in LDS; a thread reads 8 code bytes (16 columns) of one
// row, and the bf16 values go through an LDS tile (rows padded by 2 bytes)
// to be written out as rows of wt.
constexpr int kTT = 64;
// row strides of the staged tables: an odd number of 4-byte words, so that
// the 16 rows one wave reads at a time fall on distinct LDS banks
__host__ __device__ inline int tstab_stride(int64_t NG) { return static_cast<int>(NG | 1); }                   // floats
__host__ __device__ inline int tztab_stride(int64_t NG) { return 4 * static_cast<int>(((NG + 3) / 4) | 1); }  // bytes
// TILED: wt is written in the fragment-tiled layout of the prefill GEMM
// (tiled_unit in w4_internal.h) for the [K, N] matrix Wd^T (K % 128 == 0,
// N % 64 == 0): unit (k, n .. n + 7); the 64 lanes of a wave write two runs
// of 32 consecutive units.
template <bool ASYM, bool GIDX, bool TAB, bool TILED = false>
__global__ __launch_bounds__(kGThreads) void dequantize_t_kernel(DequantArgs a, uint16_t* __restrict__ wt) {
  extern __shared__ __attribute__((aligned(16))) uint8_t tsm[];
  uint16_t (*tile)[kTT + 2] = reinterpret_cast<uint16_t (*)[kTT + 2]>(tsm);     // [k][n]
  int* gsh = reinterpret_cast<int*>(tsm + kTT * (kTT + 2) * 2);                 // [64] group of column
  const int NG = static_cast<int>(a.NG);
  const int SS = tstab_stride(NG), ZS = tztab_stride(NG);
  float* stab = reinterpret_cast<float*>(gsh + kTT);                            // [64 rows][SS]
  uint8_t* ztab = reinterpret_cast<uint8_t*>(stab + kTT * SS);                  // [64 rows][ZS]
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * kTT;
  const int k0 = blockIdx.x * kTT;
  const int K = static_cast<int>(a.K);
  const int64_t KB = (a.K + 1) / 2;
  const int rows = static_cast<int>(min(static_cast<int64_t>(kTT), a.N - n0));
  // this thread's 8 code bytes (16 columns of one row), issued before the
  // tables are staged so that both latencies overlap
  const int nl = threadIdx.x >> 2, kq = (threadIdx.x & 3) * 16;
  const int kb = k0 + kq;                          // first of this thread's 16 columns
  uint32_t d[2] = {0u, 0u};
  if (nl < rows) {
    const int64_t n = n0 + nl;
    if (kb + 16 <= K && (KB & 3) == 0) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(a.codes + n * KB + kb / 2);
      d[0] = src[0];
      d[1] = src[1];
    } else {
      for (int b = 0; b < 8; ++b)
        if (kb + 2 * b < K) d[b >> 2] |= static_cast<uint32_t>(a.codes[n * KB + kb / 2 + b]) << (8 * (b & 3));
    }
  }
  for (int e = threadIdx.x; e < kTT; e += kGThreads) {
    const int k = min(k0 + e, K - 1);
    gsh[e] = GIDX ? min(max(a.g_idx[k], 0), NG - 1) : k / static_cast<int>(a.G);
  }
  if constexpr (TAB) {                             // (else the rows' tables are read from memory)
    for (int e = threadIdx.x; e < rows * NG; e += kGThreads) {
      const int r = e / NG, g = e % NG;
      const int64_t gi = (n0 + r) * a.NG + g;
      stab[r * SS + g] = a.scales[gi];
      if constexpr (ASYM) ztab[r * ZS + g] = static_cast<uint8_t>(zero_row(a.zeros, n0 + r, a.NG, a.zpk)[g]);
    }
  }
  __syncthreads();
  {
    if (nl < rows) {
      const int64_t n = n0 + nl;
      float w[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t nib = (d[e >> 3] >> (4 * (e & 7))) & 15u;
        const int gi = gsh[kq + e];
        const float sc = TAB ? stab[nl * SS + gi] : a.scales[n * a.NG + gi];
        const int zp = ASYM ? (TAB ? ztab[nl * ZS + gi] : static_cast<int>(zero_row(a.zeros, n, a.NG, a.zpk)[gi])) : 8;
        const float val = ASYM ? static_cast<float>(static_cast<int>(nib) - zp)
                               : static_cast<float>(static_cast<int>(nib ^ 8u) - 8);
        w[e] = val * sc;
      }
      // round to bf16 in pairs (v_cvt_pk_bf16_f32: nearest, ties to even) and
      // store each half in its own tile row
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const uint32_t p = __builtin_bit_cast(uint32_t, bf16x2_t{static_cast<__bf16>(w[e]), static_cast<__bf16>(w[e + 1])});
        tile[kq + e][nl] = static_cast<uint16_t>(p);
        tile[kq + e + 1][nl] = static_cast<uint16_t>(p >> 16);
      }
    }
  }
  __syncthreads();
  if constexpr (TILED) {
    const int kl = threadIdx.x % kTT, nq = (threadIdx.x / kTT) * 16;
    const int64_t k = k0 + kl;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      u32x4 q;
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = *reinterpret_cast<const uint32_t*>(&tile[kl][nq + 8 * h2 + 2 * i]);
      const int64_t unit = tiled_unit(k, n0 + nq + 8 * h2, a.N);
      // a plain store: the workspace is read back by the GEMM right after,
      // from the Infinity Cache when it is still there
      *reinterpret_cast<u32x4*>(wt + 8 * unit) = q;
    }
  } else {
    const int kl = threadIdx.x >> 2, nq = (threadIdx.x & 3) * 16;
    const int k = k0 + kl;
    if (k < K) {
      uint16_t* dst = wt + static_cast<int64_t>(k) * a.N + n0 + nq;
      const bool full = nq + 16 <= rows && (a.N & 7) == 0;
      if (full) {
        u32x4 q[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            q[h][i] = *reinterpret_cast<const uint32_t*>(&tile[kl][nq + 8 * h + 2 * i]);   // 4-byte aligned pair
        reinterpret_cast<u32x4*>(dst)[0] = q[0];
        reinterpret_cast<u32x4*>(dst)[1] = q[1];
      } else {
        for (int e = 0; e < 16; ++e)
          if (nq + e < rows) dst[e] = tile[kl][nq + e];
      }
    }
  }
}

template <bool ASYM, bool GIDX, int MT, int CPT>
hipError_t launch_split4(const GradArgs& a, int P, int rows_per, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>((a.K + kWave * CPT - 1) / (kWave * CPT)), static_cast<uint32_t>(P));
  constexpr int WV = grad_waves<MT, CPT>();
  const size_t lds = static_cast<size_t>(grad_parallel_sum<MT, CPT, WV>() ? WV : 1) * MT * CPT * kWave * sizeof(float);
  grad_split_kernel<ASYM, GIDX, MT, CPT, WV><<<grid, dim3(WV * kWave), lds, s>>>(a, rows_per);
  return hipGetLastError();
}

template <bool ASYM, bool GIDX, bool WIDE>
hipError_t launch_split3(const GradArgs& a, int P, int rows_per, hipStream_t s) {
  if (a.M <= 1) return launch_split4<ASYM, GIDX, 1, grad_cpt<1, WIDE>()>(a, P, rows_per, s);
  if (a.M <= 2) return launch_split4<ASYM, GIDX, 2, grad_cpt<2, WIDE>()>(a, P, rows_per, s);
  if (a.M <= 4) return launch_split4<ASYM, GIDX, 4, grad_cpt<4, WIDE>()>(a, P, rows_per, s);
  if (a.M <= 8) return launch_split4<ASYM, GIDX, 8, 8>(a, P, rows_per, s);
  return launch_split4<ASYM, GIDX, 16, 8>(a, P, rows_per, s);
}

}  // namespace

GradPlan grad_plan(int64_t M, int64_t N, int64_t K, int64_t G, bool has_g_idx) {
  GradPlan p{};
  if (M <= kGradSkinnyMax) {
    const int cpt = !has_g_idx && G % 32 == 0 && M <= 4 ? 32 : 8;     // columns per lane
    const int64_t cb = (K + kWave * cpt - 1) / (kWave * cpt);        // column blocks
    // about 2048 waves (two per SIMD): 256 workgroups of 8 waves (M = 1 with 32
    // columns per lane) or 512 of 4; at the decode layer's shape (K = 4096) 128
    // slices of 112 rows took 13.2-13.4 us per call against 13.6-14.1 us with
    // 256 slices of 56 rows (64, 96 and 192 slices: 17.9, 14.7, 15.5 us)
    const int wv = M <= 1 && cpt == 32 ? 8 : 4;                      // grad_waves<MT, CPT>()
    int64_t P = std::max<int64_t>(1, 2048 / wv / cb);
    P = std::min<int64_t>(P, (N + 31) / 32);                          // at least 32 rows per slice
    const int64_t per_slice = M * K * 4;
    P = std::min<int64_t>(P, std::max<int64_t>(1, kGradPartialBytes / per_slice));
    P = std::max<int64_t>(1, std::min<int64_t>(P, N));
    p.slices = static_cast<int>(P);
    p.rows_per = static_cast<int>((N + P - 1) / P);
    p.slices = static_cast<int>((N + p.rows_per - 1) / p.rows_per);
    p.workspace = static_cast<size_t>(p.slices) * static_cast<size_t>(M * K) * 4;
  } else {
    p.workspace = static_cast<size_t>(K) * static_cast<size_t>(N) * 2;
  }
  return p;
}

namespace {

// Transposed dequantize into the tiled layout with value tables: a workgroup
// owns 64 weight rows and a run of 128-column sub-tiles.  It builds once, in
// LDS, the 16 bf16 values each (row, group) can decode to (one fp32 multiply
// and one rounding each, as w4_dequantize), then per sub-tile stages the
// 64 x 64 code bytes and the columns' group offsets in LDS (double-buffered,
// the next sub-tile's loads in flight) and turns every weight into one table
// read.  A lane writes two adjacent 16-byte units of Wd^T (8 consecutive rows
// n at columns k and k + 1, the two nibbles of one code byte per row), so each
// half of a wave writes 1 KB contiguously.  Tables of up to 32 groups per row.
constexpr int kTVRows = 64;     // weight rows per workgroup
constexpr int kTVCols = 128;    // columns per sub-tile
constexpr int kTVCodeRow = 80;  // LDS bytes per staged code row (64 + 16 of padding)
constexpr int kTVMaxGroups = 32;
__host__ __device__ inline int tv_table_stride(int64_t NG) { return static_cast<int>(NG) * 32 + 4; }
size_t tv_lds_bytes(int64_t NG) {
  return static_cast<size_t>(kTVRows) * tv_table_stride(NG) + 2 * kTVRows * kTVCodeRow + 2 * kTVCols * 2;
}

template <bool ASYM, bool GIDX>
__global__ __launch_bounds__(kGThreads) void dequantize_tv_kernel(DequantArgs a, uint16_t* __restrict__ wt, int ksub) {
  extern __shared__ __attribute__((aligned(16))) uint8_t vsm[];
  const int NG = static_cast<int>(a.NG);
  const int stride = tv_table_stride(NG);
  uint8_t* vt = vsm;                                                   // [64 rows][stride]
  uint8_t* ct = vsm + kTVRows * stride;                                // [2][64 rows][kTVCodeRow]
  uint16_t* gs = reinterpret_cast<uint16_t*>(ct + 2 * kTVRows * kTVCodeRow);   // [2][128] group byte offsets
  const int t = threadIdx.x;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * kTVRows;
  const int K = static_cast<int>(a.K);
  const int64_t KB = a.K / 2;
  const int sub0 = blockIdx.x * ksub;
  const int nsub = min(ksub, K / kTVCols - sub0);

  // loads: table inputs first (they gate the build), then sub-tile 0's code
  // bytes (thread t: row t / 4, 16 bytes at 16 (t % 4)) and group indices
  const int entries = kTVRows * NG;                    // <= 64 * 32: 8 per thread
  float tsc[8];
  int tz[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = min(t + kGThreads * q, entries - 1);
    const int r = e / NG, g = e % NG;
    tsc[q] = a.scales[(n0 + r) * a.NG + g];
    tz[q] = ASYM ? static_cast<int>(zero_row(a.zeros, n0 + r, a.NG, a.zpk)[g]) : 8;
  }
  const uint8_t* crow = a.codes + (n0 + (t >> 2)) * KB + 16 * (t & 3);
  auto load_codes = [&](int sub) -> u32x4 {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow + static_cast<int64_t>(sub0 + sub) * (kTVCols / 2)));
  };
  auto load_group = [&](int sub) -> int {
    const int k = (sub0 + sub) * kTVCols + (t & (kTVCols - 1));
    return GIDX ? min(max(a.g_idx[k], 0), NG - 1) : k / static_cast<int>(a.G);
  };
  u32x4 cnext = load_codes(0);
  int gnext = load_group(0);

  // value table: entry (row r, group g, nibble u) at r * stride + 32 g + 2 u
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = t + kGThreads * q;
    if (e >= entries) break;
    const int r = e / NG, g = e % NG;
    uint32_t* dst = reinterpret_cast<uint32_t*>(vt + r * stride + 32 * g);
#pragma unroll
    for (int u = 0; u < 16; u += 2) {
      const float v0 = static_cast<float>((ASYM ? u : (u ^ 8)) - tz[q]) * tsc[q];
      const float v1 = static_cast<float>((ASYM ? u + 1 : ((u + 1) ^ 8)) - tz[q]) * tsc[q];
      dst[u / 2] = __builtin_bit_cast(uint32_t, bf16x2_t{static_cast<__bf16>(v0), static_cast<__bf16>(v1)});
    }
  }
  auto stage = [&](int buf) {
    *reinterpret_cast<u32x4*>(ct + (buf * kTVRows + (t >> 2)) * kTVCodeRow + 16 * (t & 3)) = cnext;
    if (t < kTVCols) gs[buf * kTVCols + t] = static_cast<uint16_t>(32 * gnext);
  };
  stage(0);
  if (nsub > 1) {
    cnext = load_codes(1);
    gnext = load_group(1);
  }
  __syncthreads();

  // lane (kb2, h, kp) of wave w: rows 8 c .. 8 c + 7 with c = 4 h + w (unit
  // slot w = c % 4, half h = c / 4), columns 32 kb + 2 kp and + 1 of the
  // sub-tile for the 32-column blocks kb = 2 kbt + kb2, kbt = 0, 1
  const int lane = lane_id();
  const int w = t >> 6;
  const int kb2 = lane >> 5, h = (lane >> 4) & 1, kp = lane & 15;
  const int c = 4 * h + w;
  uint32_t rbase[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) rbase[i] = static_cast<uint32_t>((8 * c + i) * stride);
  const int64_t NB = a.N / 64;
  for (int j = 0; j < nsub; ++j) {
    const int buf = j & 1;
    const uint8_t* cb = ct + buf * kTVRows * kTVCodeRow;
    const int kcol0 = (sub0 + j) * kTVCols;
#pragma unroll
    for (int kbt = 0; kbt < 2; ++kbt) {
      const int kb = 2 * kbt + kb2;
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = cb[(8 * c + i) * kTVCodeRow + 16 * kb + kp];
      const uint32_t go = *reinterpret_cast<const uint32_t*>(gs + buf * kTVCols + 32 * kb + 2 * kp);
      const uint32_t go0 = go & 0xFFFFu, go1 = go >> 16;
      uint32_t v0[8], v1[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v0[i] = *reinterpret_cast<const uint16_t*>(vt + rbase[i] + go0 + 2 * (b[i] & 15u));
        v1[i] = *reinterpret_cast<const uint16_t*>(vt + rbase[i] + go1 + 2 * (b[i] >> 4));
      }
      const int64_t kg = kcol0 + 32 * kb + 2 * kp;     // even column of the pair
      const int64_t unit = (((kg / 32) * NB + n0 / 64) * 4 + w) * 64 + 32 * h + (kg & 31);
      u32x4* dst = reinterpret_cast<u32x4*>(wt + 8 * unit);
      // plain stores: the GEMM reads the workspace right after
      dst[0] = u32x4{v0[0] | (v0[1] << 16), v0[2] | (v0[3] << 16), v0[4] | (v0[5] << 16), v0[6] | (v0[7] << 16)};
      dst[1] = u32x4{v1[0] | (v1[1] << 16), v1[2] | (v1[3] << 16), v1[4] | (v1[5] << 16), v1[6] | (v1[7] << 16)};
    }
    if (j + 1 < nsub) {
      stage(buf ^ 1);
      if (j + 2 < nsub) {
        cnext = load_codes(j + 2);
        gnext = load_group(j + 2);
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_grad_input(const GradArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  const GradPlan p = grad_plan(a.M, a.N, a.K, a.G, a.g_idx != nullptr);
  if (a.M <= kGradSkinnyMax) {
    const bool wide = !a.g_idx && a.G % 32 == 0;
    hipError_t e;
    if (a.asym) {
      e = a.g_idx ? launch_split3<true, true, false>(a, p.slices, p.rows_per, s)
          : wide  ? launch_split3<true, false, true>(a, p.slices, p.rows_per, s)
                  : launch_split3<true, false, false>(a, p.slices, p.rows_per, s);
    } else {
      e = a.g_idx ? launch_split3<false, true, false>(a, p.slices, p.rows_per, s)
          : wide  ? launch_split3<false, false, true>(a, p.slices, p.rows_per, s)
                  : launch_split3<false, false, false>(a, p.slices, p.rows_per, s);
    }
    if (e != hipSuccess) return e;
    const int64_t total = a.M * a.K;
    grad_reduce_kernel<<<dim3(static_cast<uint32_t>((total + kWave - 1) / kWave)), dim3(kRParts * kWave), 0, s>>>(
        a.partial, p.slices, total, a.dx);
    return hipGetLastError();
  }
  // transposed weight into the workspace, then the bf16 GEMM
  DequantArgs d{a.codes, a.scales, a.zeros, a.g_idx, a.N, a.K, a.G, a.NG, a.asym, nullptr, 1, a.zpk};
  uint16_t* wt = reinterpret_cast<uint16_t*>(a.partial);
  const dim3 grid(static_cast<uint32_t>((a.K + kTT - 1) / kTT), static_cast<uint32_t>((a.N + kTT - 1) / kTT));
  const size_t lds0 = kTT * (kTT + 2) * 2 + kTT * 4;
  const size_t lds = lds0 + static_cast<size_t>(kTT) * (4 * tstab_stride(a.NG) + tztab_stride(a.NG));
  if (gemm_tiled_ok(a.M, a.K, a.N) && a.K % 128 == 0 && a.N % 64 == 0 && a.NG <= kTVMaxGroups &&
      a.N / kTVRows <= 65535) {
    // Wd^T in the tiled layout through per-(row, group) value tables, then the GEMM
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const size_t tlds = tv_lds_bytes(a.NG);
    const void* kern = a.asym ? (a.g_idx ? reinterpret_cast<const void*>(dequantize_tv_kernel<true, true>)
                                         : reinterpret_cast<const void*>(dequantize_tv_kernel<true, false>))
                              : (a.g_idx ? reinterpret_cast<const void*>(dequantize_tv_kernel<false, true>)
                                         : reinterpret_cast<const void*>(dequantize_tv_kernel<false, false>));
    // the attribute is set once per kernel and device: allow the largest table
    e = ensure_lds_attribute(kern, static_cast<int>(tv_lds_bytes(kTVMaxGroups)), dev);
    if (e != hipSuccess) return e;
    // about 512 workgroups: runs of sub-tiles along K
    const int64_t subs = a.K / kTVCols, rblk = a.N / kTVRows;
    const int ksub = static_cast<int>(std::max<int64_t>(1, (subs * rblk + 511) / 512));
    const dim3 tgrid(static_cast<uint32_t>((subs + ksub - 1) / ksub), static_cast<uint32_t>(rblk));
    if (a.asym) {
      if (a.g_idx) dequantize_tv_kernel<true, true><<<tgrid, dim3(kGThreads), tlds, s>>>(d, wt, ksub);
      else dequantize_tv_kernel<true, false><<<tgrid, dim3(kGThreads), tlds, s>>>(d, wt, ksub);
    } else {
      if (a.g_idx) dequantize_tv_kernel<false, true><<<tgrid, dim3(kGThreads), tlds, s>>>(d, wt, ksub);
      else dequantize_tv_kernel<false, false><<<tgrid, dim3(kGThreads), tlds, s>>>(d, wt, ksub);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_gemm_tiled(a.dy, wt, nullptr, a.dx, a.M, a.K, a.N, s);
  }
  if (lds <= 65536 && gemm_tiled_ok(a.M, a.K, a.N) && a.K % 128 == 0 && a.N % 64 == 0) {
    // Wd^T in the tiled layout, then the GEMM that reads it straight into registers
    if (a.asym) {
      if (a.g_idx) dequantize_t_kernel<true, true, true, true><<<grid, dim3(kGThreads), lds, s>>>(d, wt);
      else dequantize_t_kernel<true, false, true, true><<<grid, dim3(kGThreads), lds, s>>>(d, wt);
    } else {
      if (a.g_idx) dequantize_t_kernel<false, true, true, true><<<grid, dim3(kGThreads), lds, s>>>(d, wt);
      else dequantize_t_kernel<false, false, true, true><<<grid, dim3(kGThreads), lds, s>>>(d, wt);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_gemm_tiled(a.dy, wt, nullptr, a.dx, a.M, a.K, a.N, s);
  }
  if (lds <= 65536) {
    if (a.asym) {
      if (a.g_idx) dequantize_t_kernel<true, true, true><<<grid, dim3(kGThreads), lds, s>>>(d, wt);
      else dequantize_t_kernel<true, false, true><<<grid, dim3(kGThreads), lds, s>>>(d, wt);
    } else {
      if (a.g_idx) dequantize_t_kernel<false, true, true><<<grid, dim3(kGThreads), lds, s>>>(d, wt);
      else dequantize_t_kernel<false, false, true><<<grid, dim3(kGThreads), lds, s>>>(d, wt);
    }
  } else {
    if (a.asym) {
      if (a.g_idx) dequantize_t_kernel<true, true, false><<<grid, dim3(kGThreads), lds0, s>>>(d, wt);
      else dequantize_t_kernel<true, false, false><<<grid, dim3(kGThreads), lds0, s>>>(d, wt);
    } else {
      if (a.g_idx) dequantize_t_kernel<false, true, false><<<grid, dim3(kGThreads), lds0, s>>>(d, wt);
      else dequantize_t_kernel<false, false, false><<<grid, dim3(kGThreads), lds0, s>>>(d, wt);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gemm_bf16(a.dy, wt, nullptr, a.dx, a.M, a.K, a.N, s);
}

}  // namespace w4
