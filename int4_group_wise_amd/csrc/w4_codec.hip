// Group-wise int4 codec kernels for gfx950: quantize + pack, and dequantize.
//
// Format and arithmetic (LoopQ packed_weight.py page: pack_weight,
// _dequantize_validated, validate; keras dense.py diff page: sub-channel int4
// with kernel_zero and g_idx):
//   codes [N, ceil(K/2)] two nibbles per byte, even column low;
//   scales [N, ceil(K/G)] fp32; zeros [N, ceil(K/G)] uint8 (zero-point mode).
//   signed:     s = max|w| / 7, q = clamp(rint(w / s), -7, 7), nibble = q & 15
//   zero-point: lo = min(0, min w), hi = max(0, max w), s = (hi - lo) / 15,
//               z = clamp(rint(-lo / s), 0, 15), q = clamp(rint(w / s) + z, 0, 15)
//   s == 0 -> s = 1.  Dequantize: fp32(value) * s, optionally rounded to bf16.
// This translation unit is compiled with -ffp-contract=off: every division is
// IEEE round-to-nearest and no multiply-add is fused, so results are
// bit-identical to the fp32 definition above.
#include <algorithm>

#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {
namespace {

constexpr int kQThreads = 256;   // one workgroup per weight row
constexpr int kDThreads = 256;

// Eight consecutive weights of one row (columns 8j .. 8j+7) as fp32; columns
// at or past K read as 0.  `e0` is the flat element index of column 8j.
template <bool BF16>
__device__ __forceinline__ void load8(const void* w, int64_t e0, int cnt, float v[8]) {
  if constexpr (BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(w) + e0;
    if (cnt == 8 && (e0 & 7) == 0) {
      const uint4 q = *reinterpret_cast<const uint4*>(p);
      const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32(d[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32(d[i] >> 16);
      }
    } else if (cnt == 8 && (e0 & 1) == 0) {
      const uint32_t* p32 = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t d = p32[i];
        v[2 * i] = bf16_to_f32(d & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32(d >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = e < cnt ? bf16_to_f32(p[e]) : 0.0f;
    }
  } else {
    const float* p = static_cast<const float*>(w) + e0;
    if (cnt == 8 && (e0 & 3) == 0) {
      const float4 a = reinterpret_cast<const float4*>(p)[0];
      const float4 b = reinterpret_cast<const float4*>(p)[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = e < cnt ? p[e] : 0.0f;
    }
  }
}

__device__ __forceinline__ float pos(float x) { return x > 0.0f ? x : 0.0f; }

// Group of a column read from g_idx, clamped into [0, NG) so that a g_idx
// violating its precondition still keeps every access in bounds.
__device__ __forceinline__ int gid_at(const int32_t* __restrict__ g_idx, int k, int NG) {
  return min(max(g_idx[k], 0), NG - 1);
}

// Per-row group statistics live in LDS as the bit patterns of non-negative
// floats, which order like unsigned integers, so an integer atomicMax is an
// exact float max:  hi[g] = max(0, max w)  (signed mode: max |w|),
//                  nlo[g] = max(0, max -w) = -min(0, min w).
template <bool ASYM, bool GIDX>
__device__ __forceinline__ void accumulate_stats(const float v[8], int k0, int cnt, int G, int NG,
                                                 const int32_t* __restrict__ g_idx,
                                                 uint32_t* hi, uint32_t* nlo) {
  if constexpr (!GIDX) {
    float m1 = 0.0f, m2 = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {   // padded columns hold 0, which changes no max
      if constexpr (ASYM) {
        m1 = fmaxf(m1, pos(v[e]));
        m2 = fmaxf(m2, pos(-v[e]));
      } else {
        m1 = fmaxf(m1, fabsf(v[e]));
      }
    }
    const int g = k0 / G;
    atomicMax(&hi[g], __float_as_uint(m1));
    if constexpr (ASYM) atomicMax(&nlo[g], __float_as_uint(m2));
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e < cnt) {
        const int g = gid_at(g_idx, k0 + e, NG);
        if constexpr (ASYM) {
          atomicMax(&hi[g], __float_as_uint(pos(v[e])));
          atomicMax(&nlo[g], __float_as_uint(pos(-v[e])));
        } else {
          atomicMax(&hi[g], __float_as_uint(fabsf(v[e])));
        }
      }
    }
  }
}

// Quantize the eight weights of a chunk and pack them into one 32-bit word
// (nibble e = column 8j + e, little-endian, so byte b holds columns 2b, 2b+1).
template <bool ASYM, bool GIDX>
__device__ __forceinline__ uint32_t quantize8(const float v[8], int k0, int cnt, int G, int NG,
                                              const int32_t* __restrict__ g_idx,
                                              const float* sc, const float* zf) {
  uint32_t packed = 0;
  const int gc = GIDX ? 0 : k0 / G;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < cnt) {
      const int g = GIDX ? gid_at(g_idx, k0 + e, NG) : gc;
      const float r = rintf(v[e] / sc[g]);
      uint32_t nib;
      if constexpr (ASYM) {
        nib = static_cast<uint32_t>(fminf(fmaxf(r + zf[g], 0.0f), 15.0f));
      } else {
        nib = static_cast<uint32_t>(static_cast<int>(fminf(fmaxf(r, -7.0f), 7.0f))) & 15u;
      }
      packed |= nib << (4 * e);
    }
  }
  return packed;
}

__device__ __forceinline__ void store_code_word(uint8_t* __restrict__ codes, int64_t off,
                                                int nbytes, uint32_t packed) {
  if (nbytes == 4 && (off & 3) == 0) {
    *reinterpret_cast<uint32_t*>(codes + off) = packed;
  } else {
    for (int b = 0; b < nbytes; ++b) codes[off + b] = static_cast<uint8_t>(packed >> (8 * b));
  }
}

// One workgroup quantizes one row.  CH > 0: each thread keeps its CH chunks of
// 8 weights in registers between the statistics pass and the packing pass
// (rows up to 2048 * CH columns).  CH == 0: longer rows, reloaded for packing.
template <bool BF16, bool ASYM, bool GIDX, int CH>
__device__ __forceinline__ void quantize_row_generic(const QuantArgs& a, int64_t n, uint32_t* lds) {
  const int NG = static_cast<int>(a.NG);
  const int K = static_cast<int>(a.K);
  const int G = static_cast<int>(a.G);
  uint32_t* hi = lds;
  uint32_t* nlo = lds + NG;
  float* sc = reinterpret_cast<float*>(lds + 2 * NG);
  float* zf = reinterpret_cast<float*>(lds + 3 * NG);
  for (int g = threadIdx.x; g < NG; g += kQThreads) { hi[g] = 0u; nlo[g] = 0u; }
  __syncthreads();

  const int nchunks = (K + 7) / 8;
  const int64_t rowoff = n * a.K;
  constexpr int CHR = CH > 0 ? CH : 1;
  float v[CHR][8];

  // pass 1: group statistics
  if constexpr (CH > 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int j = threadIdx.x + c * kQThreads;
      if (j < nchunks) {
        const int k0 = 8 * j, cnt = min(8, K - k0);
        load8<BF16>(a.w, rowoff + k0, cnt, v[c]);
        accumulate_stats<ASYM, GIDX>(v[c], k0, cnt, G, NG, a.g_idx, hi, nlo);
      }
    }
  } else {
    for (int j = threadIdx.x; j < nchunks; j += kQThreads) {
      const int k0 = 8 * j, cnt = min(8, K - k0);
      load8<BF16>(a.w, rowoff + k0, cnt, v[0]);
      accumulate_stats<ASYM, GIDX>(v[0], k0, cnt, G, NG, a.g_idx, hi, nlo);
    }
  }
  __syncthreads();

  // pass 2: scale (and zero-point) of every group of the row
  for (int g = threadIdx.x; g < NG; g += kQThreads) {
    float s, z = 0.0f;
    if constexpr (ASYM) {
      const float h = __uint_as_float(hi[g]);
      const float nl = __uint_as_float(nlo[g]);      // = -lo
      s = (h + nl) / 15.0f;                          // (hi - lo) / 15
      if (s == 0.0f) s = 1.0f;
      z = fminf(fmaxf(rintf(nl / s), 0.0f), 15.0f);  // rint(-lo / s)
      a.zeros[n * a.NG + g] = static_cast<uint8_t>(z);
    } else {
      s = __uint_as_float(hi[g]) / 7.0f;
      if (s == 0.0f) s = 1.0f;
    }
    a.scales[n * a.NG + g] = s;
    sc[g] = s;
    zf[g] = z;
  }
  __syncthreads();

  // pass 3: quantize and pack
  const int64_t KB = (a.K + 1) / 2;
  if constexpr (CH > 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int j = threadIdx.x + c * kQThreads;
      if (j < nchunks) {
        const int k0 = 8 * j, cnt = min(8, K - k0);
        const uint32_t p = quantize8<ASYM, GIDX>(v[c], k0, cnt, G, NG, a.g_idx, sc, zf);
        store_code_word(a.codes, n * KB + 4 * j, min(4, static_cast<int>(KB) - 4 * j), p);
      }
    }
  } else {
    for (int j = threadIdx.x; j < nchunks; j += kQThreads) {
      const int k0 = 8 * j, cnt = min(8, K - k0);
      load8<BF16>(a.w, rowoff + k0, cnt, v[0]);
      const uint32_t p = quantize8<ASYM, GIDX>(v[0], k0, cnt, G, NG, a.g_idx, sc, zf);
      store_code_word(a.codes, n * KB + 4 * j, min(4, static_cast<int>(KB) - 4 * j), p);
    }
  }
}

template <bool BF16, bool ASYM, bool GIDX, int CH>
__global__ __launch_bounds__(kQThreads) void quantize_pack_kernel(QuantArgs a) {
  extern __shared__ uint32_t lds[];
  quantize_row_generic<BF16, ASYM, GIDX, CH>(a, blockIdx.x, lds);
}

// Largest row table (scales + zero-points) the act-order dequantizer stages
// in LDS; rows with more groups gather from global memory instead.
constexpr int64_t kDequantLdsGroups = 8192;

// Dequantize: one thread per 8 consecutive columns of one row.  GIDX: 0 =
// contiguous groups, 1 = act-order with the row's scale / zero-point table
// staged in LDS (g_idx read 8 entries at a time), 2 = act-order gathering the
// table entries from global memory.
template <bool OUT_BF16, bool ASYM, int GIDX>
__global__ __launch_bounds__(kDThreads) void dequantize_kernel(DequantArgs a, int chunk_blocks) {
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  const int64_t n = blockIdx.x / chunk_blocks;
  const int j = (blockIdx.x % chunk_blocks) * kDThreads + threadIdx.x;
  const int K = static_cast<int>(a.K);
  const int nchunks = (K + 7) / 8;
  const int NG = static_cast<int>(a.NG);
  float* st = reinterpret_cast<float*>(dsm);
  uint8_t* zt = dsm + 4 * NG;
  if constexpr (GIDX == 1) {
    for (int g = threadIdx.x; g < NG; g += kDThreads) {
      st[g] = a.scales[n * a.NG + g];
      if constexpr (ASYM) zt[g] = static_cast<uint8_t>(zero_row(a.zeros, n, a.NG, a.zpk)[g]);
    }
    __syncthreads();
  }
  if (j >= nchunks) return;
  const int64_t KB = (a.K + 1) / 2;
  const int k0 = 8 * j, cnt = min(8, K - k0);

  const int64_t coff = n * KB + 4 * j;
  uint32_t d = 0;
  if (cnt == 8 && (coff & 3) == 0) {
    d = *reinterpret_cast<const uint32_t*>(a.codes + coff);
  } else {
    const int nb = (cnt + 1) / 2;
    for (int b = 0; b < nb; ++b) d |= static_cast<uint32_t>(a.codes[coff + b]) << (8 * b);
  }

  float o[8];
  const float* srow = a.scales + n * a.NG;
  const ZeroRow zrow = zero_row(ASYM ? a.zeros : nullptr, n, a.NG, a.zpk);
  if constexpr (GIDX == 0) {
    const int g = k0 / static_cast<int>(a.G);
    const float s = srow[g];
    const int z = ASYM ? static_cast<int>(zrow[g]) : 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int nib = static_cast<int>((d >> (4 * e)) & 15u);
      const int val = ASYM ? nib - z : (nib ^ 8) - 8;
      o[e] = static_cast<float>(val) * s;
    }
  } else if constexpr (GIDX == 1) {
    int gv[8];
    if (cnt == 8) {
      const u32x4 g0 = *reinterpret_cast<const u32x4*>(a.g_idx + k0);
      const u32x4 g1 = *reinterpret_cast<const u32x4*>(a.g_idx + k0 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { gv[e] = static_cast<int>(g0[e]); gv[4 + e] = static_cast<int>(g1[e]); }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gv[e] = e < cnt ? a.g_idx[k0 + e] : 0;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int g = min(max(gv[e], 0), NG - 1);
      const int nib = static_cast<int>((d >> (4 * e)) & 15u);
      const int val = ASYM ? nib - static_cast<int>(zt[g]) : (nib ^ 8) - 8;
      o[e] = static_cast<float>(val) * st[g];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[e] = 0.0f;
      if (e < cnt) {
        const int g = gid_at(a.g_idx, k0 + e, NG);
        const int nib = static_cast<int>((d >> (4 * e)) & 15u);
        const int val = ASYM ? nib - static_cast<int>(zrow[g]) : (nib ^ 8) - 8;
        o[e] = static_cast<float>(val) * srow[g];
      }
    }
  }

  const int64_t e0 = n * a.K + k0;
  if constexpr (OUT_BF16) {
    uint16_t* out = static_cast<uint16_t*>(a.out) + e0;
    if (cnt == 8 && (e0 & 7) == 0) {
      uint4 q;
      q.x = f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16);
      q.y = f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16);
      q.z = f32_to_bf16(o[4]) | (f32_to_bf16(o[5]) << 16);
      q.w = f32_to_bf16(o[6]) | (f32_to_bf16(o[7]) << 16);
      *reinterpret_cast<uint4*>(out) = q;
    } else if (cnt == 8 && (e0 & 1) == 0) {
      uint32_t* o32 = reinterpret_cast<uint32_t*>(out);
#pragma unroll
      for (int i = 0; i < 4; ++i) o32[i] = f32_to_bf16(o[2 * i]) | (f32_to_bf16(o[2 * i + 1]) << 16);
    } else {
      for (int e = 0; e < cnt; ++e) out[e] = static_cast<uint16_t>(f32_to_bf16(o[e]));
    }
  } else {
    float* out = static_cast<float*>(a.out) + e0;
    if (cnt == 8 && (e0 & 3) == 0) {
      reinterpret_cast<float4*>(out)[0] = make_float4(o[0], o[1], o[2], o[3]);
      reinterpret_cast<float4*>(out)[1] = make_float4(o[4], o[5], o[6], o[7]);
    } else {
      for (int e = 0; e < cnt; ++e) out[e] = o[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Row quantizer for contiguous groups, G a power of two in [8, 512], rows of
// 64 .. 8 * 8 * kQThreads columns.  One 256-thread workgroup per row; thread
// t holds chunks t, t + 256, ... (eight columns each) in registers, so a
// group is G / 8 consecutive lanes of one wave and its statistics are a lane
// reduction (no LDS, no barrier).
//
// Loads.  A row starts OB = (n K es) mod 16 bytes past a 16-byte boundary.
// OB is the same for the whole workgroup and selects a straight-line variant
// that reads aligned 16-byte segments and shifts them into place.  A chunk's
// segments can reach up to 48 bytes into the next row, so the last row of
// the matrix is read element by element instead.
//
// Statistics, division and packing of a chunk: quantize_chunk8 (w4_device.h).
// ---------------------------------------------------------------------------

// The eight weights of chunk j (columns 8j .. 8j+7) of a row whose first byte
// sits OB bytes past the 16-byte aligned pointer `rowA`.  OB < 0: element
// loads from `row` (cnt valid columns).
template <bool BF16, int OB>
struct ChunkLoader {
  static constexpr int kCB = BF16 ? 16 : 32;                 // bytes per chunk
  static constexpr int kNS = kCB / 16 + (OB > 0 ? 1 : 0);    // aligned segments
  u32x4 seg[kNS];
  __device__ __forceinline__ void issue(const uint8_t* __restrict__ rowA, int j) {
#pragma unroll
    for (int s = 0; s < kNS; ++s)   // weights are read once: non-temporal
      seg[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowA + kCB * j + 16 * s));
  }
  __device__ __forceinline__ void unpack(float v[8]) const {
    uint32_t d[4 * kNS];
#pragma unroll
    for (int s = 0; s < kNS; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) d[4 * s + i] = seg[s][i];
    constexpr int q = (OB > 0 ? OB : 0) / 4, r = (OB > 0 ? OB : 0) % 4;
    uint32_t w[kCB / 4];
#pragma unroll
    for (int k = 0; k < kCB / 4; ++k) w[k] = r == 0 ? d[q + k] : __builtin_amdgcn_alignbyte(d[q + k + 1], d[q + k], r);
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
    }
  }
};

template <bool BF16, bool ASYM, int CH, int OB>
__device__ __forceinline__ void quantize_row(const QuantArgs& a, int64_t n, int lpg) {
  constexpr int kEs = BF16 ? 2 : 4;
  const int K = static_cast<int>(a.K);
  const int nchunks = (K + 7) / 8;
  const int lane = lane_id();

  // phase 1: every load of the thread in flight before any use
  float v[CH][8];
  if constexpr (OB >= 0) {
    const uint8_t* rowA = static_cast<const uint8_t*>(a.w) + n * a.K * kEs - OB;
    ChunkLoader<BF16, OB> ld[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) ld[c].issue(rowA, min(static_cast<int>(threadIdx.x) + c * kQThreads, nchunks - 1));
#pragma unroll
    for (int c = 0; c < CH; ++c) ld[c].unpack(v[c]);
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int k0 = 8 * min(static_cast<int>(threadIdx.x) + c * kQThreads, nchunks - 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = min(k0 + e, K - 1);
        v[c][e] = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(a.w)[n * a.K + k])
                       : static_cast<const float*>(a.w)[n * a.K + k];
      }
    }
  }

  const int64_t KB = (a.K + 1) / 2;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j = static_cast<int>(threadIdx.x) + c * kQThreads;
    const int cnt = K - 8 * j;                 // valid columns of the chunk (> 8: all)
    if (cnt < 8) {                             // row tail and idle lanes hold zeros
#pragma unroll
      for (int e = 0; e < 8; ++e) v[c][e] = e < cnt ? v[c][e] : 0.0f;
    }
    float sc, zf;
    const uint32_t packed = quantize_chunk8<ASYM>(v[c], cnt, lpg, sc, zf);
    if (cnt <= 0) continue;
    const int g = j / lpg;
    if ((lane & (lpg - 1)) == 0) {
      a.scales[n * a.NG + g] = sc;
      if constexpr (ASYM) a.zeros[n * a.NG + g] = static_cast<uint8_t>(zf);
    }
    store_code_word(a.codes, n * KB + 4 * j, min(4, static_cast<int>(KB) - 4 * j), packed);
  }
}

template <bool BF16, bool ASYM, int CH>
__global__ __launch_bounds__(kQThreads) void quantize_rows_kernel(QuantArgs a, int lpg) {
  const int64_t n = blockIdx.x;
  if (n == a.N - 1) {
    quantize_row<BF16, ASYM, CH, -1>(a, n, lpg);
    return;
  }
  const int ob = static_cast<int>((n * a.K * (BF16 ? 2 : 4)) & 15);
  if constexpr (BF16) {
    switch (ob) {
      case 0: quantize_row<BF16, ASYM, CH, 0>(a, n, lpg); break;
      case 2: quantize_row<BF16, ASYM, CH, 2>(a, n, lpg); break;
      case 4: quantize_row<BF16, ASYM, CH, 4>(a, n, lpg); break;
      case 6: quantize_row<BF16, ASYM, CH, 6>(a, n, lpg); break;
      case 8: quantize_row<BF16, ASYM, CH, 8>(a, n, lpg); break;
      case 10: quantize_row<BF16, ASYM, CH, 10>(a, n, lpg); break;
      case 12: quantize_row<BF16, ASYM, CH, 12>(a, n, lpg); break;
      default: quantize_row<BF16, ASYM, CH, 14>(a, n, lpg); break;
    }
  } else {
    switch (ob) {
      case 0: quantize_row<BF16, ASYM, CH, 0>(a, n, lpg); break;
      case 4: quantize_row<BF16, ASYM, CH, 4>(a, n, lpg); break;
      case 8: quantize_row<BF16, ASYM, CH, 8>(a, n, lpg); break;
      default: quantize_row<BF16, ASYM, CH, 12>(a, n, lpg); break;
    }
  }
}

template <bool BF16, bool ASYM>
hipError_t launch_qrows(const QuantArgs& a, hipStream_t s) {
  const int lpg = static_cast<int>(a.G / 8);
  const int64_t nchunks = (a.K + 7) / 8;
  const dim3 grid(static_cast<uint32_t>(a.N)), block(kQThreads);
  if (nchunks <= 1 * kQThreads) quantize_rows_kernel<BF16, ASYM, 1><<<grid, block, 0, s>>>(a, lpg);
  else if (nchunks <= 2 * kQThreads) quantize_rows_kernel<BF16, ASYM, 2><<<grid, block, 0, s>>>(a, lpg);
  else if (nchunks <= 4 * kQThreads) quantize_rows_kernel<BF16, ASYM, 4><<<grid, block, 0, s>>>(a, lpg);
  else quantize_rows_kernel<BF16, ASYM, 8><<<grid, block, 0, s>>>(a, lpg);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Act-order quantizer for a g_idx whose groups all hold exactly G columns (G a
// power of two in [8, 512], K <= 8192): a workgroup sorts the columns by group
// once (counting sort of g_idx in LDS), then for each of its kActQRows rows
// stages the row in LDS as fp32 and reads it in group order, so that a group
// is G / 8 consecutive lanes of eight columns and the lane-reduction
// quantizer applies; the codes return to column order through an LDS byte
// table and are packed and written coalesced.  The order of the columns
// within a group does not matter (the statistics are maxima, the codes are
// per column), so the results are deterministic.  If the groups turn out not
// to be uniform, the workgroup quantizes its rows with the general per-row
// algorithm instead (every workgroup sees the same g_idx).
// ---------------------------------------------------------------------------
constexpr int kActQRows = 4;   // rows per workgroup (measured best of 1, 2, 4, 8, 16)
constexpr int kActQMaxK = 8192;

__host__ __device__ inline size_t act_q_lds(int64_t K, int64_t NG) {
  const size_t fast = ((4 * NG + 15) & ~15) + ((2 * K + 15) & ~15) + 4 * K + ((K + 15) & ~15);
  const size_t slow = static_cast<size_t>(NG) * 4 * sizeof(uint32_t);
  return fast > slow ? fast : slow;
}

template <bool BF16, bool ASYM>
__global__ __launch_bounds__(kQThreads) void quantize_act_kernel(QuantArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t qsm[];
  __shared__ int uniform;
  const int K = static_cast<int>(a.K);
  const int NG = static_cast<int>(a.NG);
  const int G = static_cast<int>(a.G);
  const int lpg = G / 8;
  const int lane = lane_id();
  int* cnt = reinterpret_cast<int*>(qsm);                                       // [NG]
  uint16_t* perm = reinterpret_cast<uint16_t*>(qsm + ((4 * NG + 15) & ~15));    // [K] column of sorted position
  float* rowv = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(perm) + ((2 * K + 15) & ~15));  // [K]
  uint8_t* cbt = reinterpret_cast<uint8_t*>(rowv + K);                          // [K] code of column

  // group sizes; uniform iff every group holds exactly G columns
  for (int g = threadIdx.x; g < NG; g += kQThreads) cnt[g] = 0;
  if (threadIdx.x == 0) uniform = 1;
  __syncthreads();
  for (int k = threadIdx.x; k < K; k += kQThreads) atomicAdd(&cnt[gid_at(a.g_idx, k, NG)], 1);
  __syncthreads();
  for (int g = threadIdx.x; g < NG; g += kQThreads)
    if (cnt[g] != G) uniform = 0;
  __syncthreads();
  const int64_t nb = static_cast<int64_t>(blockIdx.x) * kActQRows;
  if (!uniform) {
    for (int r = 0; r < kActQRows; ++r) {
      if (nb + r >= a.N) break;                    // uniform
      __syncthreads();                             // the previous row is done with the tables
      quantize_row_generic<BF16, ASYM, true, kActQMaxK / 8 / kQThreads>(a, nb + r, reinterpret_cast<uint32_t*>(qsm));
    }
    return;
  }
  // sorted positions: group g holds positions g G .. g G + G - 1
  for (int g = threadIdx.x; g < NG; g += kQThreads) cnt[g] = g * G;
  __syncthreads();
  for (int k = threadIdx.x; k < K; k += kQThreads) perm[atomicAdd(&cnt[gid_at(a.g_idx, k, NG)], 1)] = static_cast<uint16_t>(k);

  constexpr int kEs = BF16 ? 2 : 4;
  constexpr int kSegMax = kActQMaxK * kEs / 16 / kQThreads;   // 16-byte row segments per thread
  constexpr int kChMax = kActQMaxK / 8 / kQThreads;           // 8-column chunks per thread
  const int nseg = K * kEs / 16;
  const int nch = K / 8;
  const int64_t KB = a.K / 2;
  // rows are software-pipelined: the next row's loads are in flight while
  // the current row is quantized and packed (read once: non-temporal)
  u32x4 seg[kSegMax];
  auto load_row = [&](int64_t n) {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.w) + n * a.K * kEs);
#pragma unroll
    for (int i = 0; i < kSegMax; ++i) {
      const int sg = threadIdx.x + kQThreads * i;
      if (sg < nseg) seg[i] = __builtin_nontemporal_load(src + sg);
    }
  };
  if (nb < a.N) load_row(nb);
  for (int r = 0; r < kActQRows; ++r) {
    const int64_t n = nb + r;
    if (n >= a.N) break;                           // uniform
    // the row into LDS as fp32 (the previous row's reads of it are done:
    // barrier after its quantization)
#pragma unroll
    for (int i = 0; i < kSegMax; ++i) {
      const int sg = threadIdx.x + kQThreads * i;
      if (sg < nseg) {
        if constexpr (BF16) {
          f32x4_t lo, hi;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            lo[2 * j] = __uint_as_float(seg[i][j] << 16);
            lo[2 * j + 1] = __uint_as_float(seg[i][j] & 0xFFFF0000u);
            hi[2 * j] = __uint_as_float(seg[i][2 + j] << 16);
            hi[2 * j + 1] = __uint_as_float(seg[i][2 + j] & 0xFFFF0000u);
          }
          reinterpret_cast<f32x4_t*>(rowv)[2 * sg] = lo;
          reinterpret_cast<f32x4_t*>(rowv)[2 * sg + 1] = hi;
        } else {
          reinterpret_cast<u32x4*>(rowv)[sg] = seg[i];
        }
      }
    }
    __syncthreads();                               // row staged (and, for the first row, perm built)
    if (r + 1 < kActQRows && n + 1 < a.N) load_row(n + 1);
    // quantize in group order: chunk c = sorted positions 8c .. 8c + 7, group 8c / G
#pragma unroll
    for (int i = 0; i < kChMax; ++i) {
      const int c = threadIdx.x + kQThreads * i;
      if (i * kQThreads >= nch) break;             // uniform; within a pass idle lanes form whole groups
      float v[8];
      int col[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        col[e] = c < nch ? perm[8 * c + e] : 0;
        v[e] = c < nch ? rowv[col[e]] : 0.0f;
      }
      float sc, zf;
      const uint32_t packed = quantize_chunk8<ASYM>(v, c < nch ? 8 : 0, lpg, sc, zf);
      if (c < nch) {
#pragma unroll
        for (int e = 0; e < 8; ++e) cbt[col[e]] = static_cast<uint8_t>((packed >> (4 * e)) & 15u);
        if ((lane & (lpg - 1)) == 0) {
          const int g = (8 * c) / G;
          a.scales[n * a.NG + g] = sc;
          if constexpr (ASYM) a.zeros[n * a.NG + g] = static_cast<uint8_t>(zf);
        }
      }
    }
    __syncthreads();                               // codes of the row complete in column order
    // pack 8 columns per thread into one code word
#pragma unroll
    for (int i = 0; i < kChMax; ++i) {
      const int j = threadIdx.x + kQThreads * i;
      if (j < nch) {
        const u32x2 b = *reinterpret_cast<const u32x2*>(cbt + 8 * j);
        const uint32_t lo = b[0] | (b[0] >> 4), hi = b[1] | (b[1] >> 4);   // nibble pairs at bytes 0 and 2
        const uint32_t w = (lo & 0xFFu) | ((lo >> 8) & 0xFF00u) | ((hi & 0xFFu) << 16) | (((hi >> 8) & 0xFF00u) << 16);
        __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(a.codes + n * KB) + j);
      }
    }
  }
}

template <bool BF16, bool ASYM>
hipError_t launch_qact(const QuantArgs& a, hipStream_t s) {
  const size_t lds = act_q_lds(a.K, a.NG);
  const dim3 grid(static_cast<uint32_t>((a.N + kActQRows - 1) / kActQRows)), block(kQThreads);
  quantize_act_kernel<BF16, ASYM><<<grid, block, lds, s>>>(a);
  return hipGetLastError();
}

template <bool BF16, bool ASYM, bool GIDX>
hipError_t launch_q3(const QuantArgs& a, hipStream_t s) {
  const size_t lds = static_cast<size_t>(a.NG) * 4 * sizeof(uint32_t);
  const int64_t nchunks = (a.K + 7) / 8;
  const dim3 grid(static_cast<uint32_t>(a.N)), block(kQThreads);
  if (nchunks <= 1 * kQThreads)
    quantize_pack_kernel<BF16, ASYM, GIDX, 1><<<grid, block, lds, s>>>(a);
  else if (nchunks <= 2 * kQThreads)
    quantize_pack_kernel<BF16, ASYM, GIDX, 2><<<grid, block, lds, s>>>(a);
  else if (nchunks <= 4 * kQThreads)
    quantize_pack_kernel<BF16, ASYM, GIDX, 4><<<grid, block, lds, s>>>(a);
  else if (nchunks <= 8 * kQThreads)
    quantize_pack_kernel<BF16, ASYM, GIDX, 8><<<grid, block, lds, s>>>(a);
  else
    quantize_pack_kernel<BF16, ASYM, GIDX, 0><<<grid, block, lds, s>>>(a);
  return hipGetLastError();
}

template <bool BF16, bool ASYM>
hipError_t launch_q2(const QuantArgs& a, hipStream_t s) {
  const bool pow2 = (a.G & (a.G - 1)) == 0;
  if (a.g_idx) {
    // act-order: group-sorted rows when the groups can be uniform and the
    // tables fit in LDS (the kernel checks the g_idx itself)
    if (pow2 && a.G >= 8 && a.G <= 512 && a.K <= kActQMaxK && a.K % a.G == 0 && act_q_lds(a.K, a.NG) <= 65536)
      return launch_qact<BF16, ASYM>(a, s);
    return launch_q3<BF16, ASYM, true>(a, s);
  }
  // fast path: contiguous power-of-two groups of at most 512 columns, rows
  // of at most 2048 * 8 columns
  if (pow2 && a.G >= 8 && a.G <= 512 && a.K >= 64 && a.K <= 8 * 8 * kQThreads) return launch_qrows<BF16, ASYM>(a, s);
  return launch_q3<BF16, ASYM, false>(a, s);
}

// ---------------------------------------------------------------------------
// Row dequantizer for contiguous power-of-two groups and rows of at least
// 1024 columns; one workgroup per row.  Lane l of a wave decodes column chunk
// i = B + l - 1 (eight columns from a multiple of 8: one code dword, one
// group).  The output is written in the 16-byte chunks of the flattened
// [N, K] array: output chunk i of the row holds its last SFT columns of
// column chunk i - 1 and the first 8 - SFT of chunk i, SFT = (n K) mod 8 being
// the same for the whole row, so each lane takes the words it needs from its
// left neighbour (one-lane wave shift) and funnel-shifts them into place.
// Lane 0 only feeds lane 1: a wave step writes 63 output chunks.  The first
// and last output chunks of a row are shared with the neighbouring rows and
// are written element by element (each row writes only its own elements).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
constexpr int kWaveShr1 = 0x138;   // lane l receives lane l - 1

template <bool OUT_BF16, bool ASYM, int SFT>
__device__ __forceinline__ void dequantize_row(const DequantArgs& a, int64_t n, int lg) {
  const int K = static_cast<int>(a.K);
  const int nch = (K + 7) / 8;                       // column chunks of the row
  const int J = (K - 1 + SFT) / 8 + 1;              // output chunks touching the row
  const int64_t e0 = n * a.K;
  const int64_t f0 = e0 >> 3;
  const int64_t KB = (a.K + 1) / 2;
  const int64_t cb = n * KB;                         // row's first code byte
  const int cadj = static_cast<int>(cb & 3);
  const uint8_t* cbase = a.codes + (cb - cadj);
  const int64_t total = a.N * KB;
  const bool last = n == a.N - 1;
  const float* srow = a.scales + n * a.NG;
  const ZeroRow zrow = zero_row(ASYM ? a.zeros : nullptr, n, a.NG, a.zpk);
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  constexpr int kWaves = kDThreads / kWave;
  const uint32_t bmask = byte_nibble_mask();

  for (int B = 63 * wave; B < J; B += 63 * kWaves) {
    const int i = B + lane - 1;
    const int ic = min(max(i, 0), nch - 1);
    // the chunk's code word (bytes 4 ic .. 4 ic + 3 of the row)
    uint32_t d;
    if (!last) {
      const uint32_t d0 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(cbase + 4 * ic));
      d = d0;
      if (cadj) d = __builtin_amdgcn_alignbyte(*reinterpret_cast<const uint32_t*>(cbase + 4 * ic + 4), d0, cadj);
    } else {                                         // stay inside the buffer
      d = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        d |= static_cast<uint32_t>(a.codes[min(cb + 4 * ic + b, total - 1)]) << (8 * b);
    }
    const int g = (8 * ic) >> lg;
    const float s = srow[g];
    float o[8];
    if constexpr (ASYM) {
      const float z = static_cast<float>(zrow[g]);
      const uint32_t lo = d & bmask, hi = (d >> 4) & bmask;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = (static_cast<float>((((e & 1) ? hi : lo) >> (8 * (e >> 1))) & 0xFFu) - z) * s;
    } else {
      // u = q + 8 in [0, 15]; fma(u, s, -8 s) rounds (u - 8) s once, as the
      // plain product does (-8 s is exact unless it overflows)
      d ^= 0x88888888u;
      const uint32_t lo = d & bmask, hi = (d >> 4) & bmask;
      const float m8 = -8.0f * s;
      if (fabsf(m8) < __builtin_inff()) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[e] = __builtin_fmaf(static_cast<float>((((e & 1) ? hi : lo) >> (8 * (e >> 1))) & 0xFFu), s, m8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[e] = (static_cast<float>((((e & 1) ? hi : lo) >> (8 * (e >> 1))) & 0xFFu) - 8.0f) * s;
      }
    }

    // words of column chunk i, then those of chunk i - 1 from the left lane
    constexpr int kW = OUT_BF16 ? 4 : 8;             // 32-bit words per chunk
    uint32_t P[kW], C[2 * kW];
    if constexpr (OUT_BF16) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x2_t p = {static_cast<__bf16>(o[2 * k]), static_cast<__bf16>(o[2 * k + 1])};
        P[k] = __builtin_bit_cast(uint32_t, p);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) P[k] = __float_as_uint(o[k]);
    }
    // output element m = concatenated element (8 - SFT + m) of [chunk i-1 | chunk i]
    constexpr int kByte = (8 - SFT) * (OUT_BF16 ? 2 : 4);   // byte offset into the 2 kW words
    constexpr int kW0 = kByte / 4, kR = kByte % 4;
#pragma unroll
    for (int k = 0; k < kW; ++k) C[kW + k] = P[k];
#pragma unroll
    for (int k = 0; k < kW; ++k) C[k] = k >= kW0 ? dpp_u32<kWaveShr1>(P[k]) : 0u;
    uint32_t out[kW];
#pragma unroll
    for (int k = 0; k < kW; ++k)
      out[k] = kR == 0 ? C[kW0 + k] : __builtin_amdgcn_alignbyte(C[kW0 + k + 1], C[kW0 + k], kR);

    const int j = i;                                 // output chunk written by this lane
    if (lane == 0 || j >= J) continue;
    const int c0 = 8 * j - SFT;                      // column of its element 0
    if (c0 >= 0 && c0 + 8 <= K) {
      if constexpr (OUT_BF16) {
        __builtin_nontemporal_store(u32x4{out[0], out[1], out[2], out[3]},   // streamed out once
                                    reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + 8 * (f0 + j)));
      } else {
        u32x4* dst = reinterpret_cast<u32x4*>(static_cast<float*>(a.out) + 8 * (f0 + j));
        dst[0] = u32x4{out[0], out[1], out[2], out[3]};
        dst[1] = u32x4{out[4], out[5], out[6], out[7]};
      }
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int col = c0 + m;
        if (col >= 0 && col < K) {
          if constexpr (OUT_BF16) static_cast<uint16_t*>(a.out)[e0 + col] = static_cast<uint16_t>(out[m / 2] >> (16 * (m & 1)));
          else static_cast<uint32_t*>(a.out)[e0 + col] = out[m];
        }
      }
    }
  }
}

template <bool OUT_BF16, bool ASYM>
__global__ __launch_bounds__(kDThreads) void dequantize_rows_kernel(DequantArgs a, int lg) {
  const int64_t n = blockIdx.x;
  switch (static_cast<int>((n * a.K) & 7)) {
    case 0: dequantize_row<OUT_BF16, ASYM, 0>(a, n, lg); break;
    case 1: dequantize_row<OUT_BF16, ASYM, 1>(a, n, lg); break;
    case 2: dequantize_row<OUT_BF16, ASYM, 2>(a, n, lg); break;
    case 3: dequantize_row<OUT_BF16, ASYM, 3>(a, n, lg); break;
    case 4: dequantize_row<OUT_BF16, ASYM, 4>(a, n, lg); break;
    case 5: dequantize_row<OUT_BF16, ASYM, 5>(a, n, lg); break;
    case 6: dequantize_row<OUT_BF16, ASYM, 6>(a, n, lg); break;
    default: dequantize_row<OUT_BF16, ASYM, 7>(a, n, lg); break;
  }
}

// ---------------------------------------------------------------------------
// Act-order dequantizer.  A workgroup owns kActRows rows x 2048 columns.  It
// first builds, for each (row, group), the 16 possible outputs of that group
// (value(u) * s rounded to the output type) as a table in LDS; then each
// thread takes 8 columns, loads their 8 group indices once, and for each of
// the rows turns every nibble into one table lookup.  The group indices are
// read once per 16 rows instead of once per row, and the per-weight work is a
// shift, a mask and an LDS read.
// ---------------------------------------------------------------------------
constexpr int kActRows = 8;

template <bool OUT_BF16>
__host__ __device__ constexpr int act_entry_bytes() { return OUT_BF16 ? 2 : 4; }

// rows of table a workgroup can hold for NG groups in 64 KB of LDS (0: none)
template <bool OUT_BF16>
__host__ __device__ inline int act_rows(int64_t NG) {
  const int64_t per_row = NG * 16 * act_entry_bytes<OUT_BF16>();
  const int64_t r = 65536 / per_row;
  return static_cast<int>(r >= kActRows ? kActRows : r);
}

template <bool OUT_BF16, bool ASYM>
__global__ __launch_bounds__(kDThreads) void dequantize_act_kernel(DequantArgs a, int rows) {
  extern __shared__ __attribute__((aligned(16))) uint8_t tsm[];
  constexpr int kEB = act_entry_bytes<OUT_BF16>();
  const int NG = static_cast<int>(a.NG);
  const int K = static_cast<int>(a.K);
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * rows;
  const int nrows = static_cast<int>(min(static_cast<int64_t>(rows), a.N - row0));

  // 1. this thread's 8 columns (chunk j): group offsets and every row's code
  //    word, loaded before the table is built so that both latencies overlap
  const int j = blockIdx.x * kDThreads + threadIdx.x;
  const int k0 = 8 * j;
  const bool live = k0 < K;
  const int cnt = live ? min(8, K - k0) : 0;
  // byte offset of each column's group inside a row's table
  uint32_t goff[8];
  if (!live) {
#pragma unroll
    for (int e = 0; e < 8; ++e) goff[e] = 0;
  } else if (cnt == 8) {
    const u32x4 g0 = *reinterpret_cast<const u32x4*>(a.g_idx + k0);
    const u32x4 g1 = *reinterpret_cast<const u32x4*>(a.g_idx + k0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      goff[e] = static_cast<uint32_t>(min(max(static_cast<int>(g0[e]), 0), NG - 1)) * 16 * kEB;
      goff[4 + e] = static_cast<uint32_t>(min(max(static_cast<int>(g1[e]), 0), NG - 1)) * 16 * kEB;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      goff[e] = static_cast<uint32_t>(min(max(a.g_idx[min(k0 + e, K - 1)], 0), NG - 1)) * 16 * kEB;
  }

  const int64_t KB = (a.K + 1) / 2;
  // every row's code word first (in flight together), then the lookups
  uint32_t dw[kActRows];
  if (cnt == 8 && (KB & 3) == 0) {               // aligned words; rows past the end reload the last
#pragma unroll
    for (int r = 0; r < kActRows; ++r)
      dw[r] = *reinterpret_cast<const uint32_t*>(a.codes + (row0 + min(r, nrows - 1)) * KB + 4 * j);
  } else {
#pragma unroll
    for (int r = 0; r < kActRows; ++r) {
      dw[r] = 0;
      if (live && r < nrows) {
        const int64_t off = (row0 + r) * KB + 4 * j;
        for (int b = 0; b < (cnt + 1) / 2; ++b) dw[r] |= static_cast<uint32_t>(a.codes[off + b]) << (8 * b);
      }
    }
  }
  // 2. table: entry (r, g, u) at byte ((r * NG + g) * 16 + u) * kEB
  for (int p = threadIdx.x; p < nrows * NG; p += kDThreads) {
    const int64_t gi = (row0 + p / NG) * a.NG + p % NG;
    const float s = a.scales[gi];
    const int z = ASYM ? static_cast<int>(zero_row(a.zeros, row0 + p / NG, a.NG, a.zpk)[p % NG]) : 8;
    uint32_t wv[16 * kEB / 4];
#pragma unroll
    for (int u = 0; u < 16; u += 2) {
      // signed codes: nibble u holds q with u = q & 15, value (u ^ 8) - 8.
      // The value is formed in integers (a float 0 - z may be folded to -z,
      // which gives -0 for z = 0)
      const float v0 = static_cast<float>((ASYM ? u : (u ^ 8)) - z) * s;
      const float v1 = static_cast<float>((ASYM ? u + 1 : ((u + 1) ^ 8)) - z) * s;
      if constexpr (OUT_BF16) {
        wv[u / 2] = f32_to_bf16(v0) | (f32_to_bf16(v1) << 16);
      } else {
        wv[u] = __float_as_uint(v0);
        wv[u + 1] = __float_as_uint(v1);
      }
    }
    u32x4* dst = reinterpret_cast<u32x4*>(tsm + static_cast<size_t>(p) * 16 * kEB);
#pragma unroll
    for (int q = 0; q < 16 * kEB / 16; ++q) dst[q] = u32x4{wv[4 * q], wv[4 * q + 1], wv[4 * q + 2], wv[4 * q + 3]};
  }
  __syncthreads();

  if (!live) return;
#pragma unroll
  for (int r = 0; r < kActRows; ++r) {
    if (r >= nrows) break;
    const uint8_t* trow = tsm + static_cast<size_t>(r) * NG * 16 * kEB;
    const int64_t e0 = (row0 + r) * a.K + k0;
    uint32_t o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t u = (dw[r] >> (4 * e)) & 15u;
      o[e] = OUT_BF16 ? *reinterpret_cast<const uint16_t*>(trow + goff[e] + 2 * u)
                      : *reinterpret_cast<const uint32_t*>(trow + goff[e] + 4 * u);
    }
    if constexpr (OUT_BF16) {
      uint16_t* out = static_cast<uint16_t*>(a.out) + e0;
      if (cnt == 8 && (e0 & 7) == 0) {
        *reinterpret_cast<u32x4*>(out) = u32x4{o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16)};
      } else {
        for (int e = 0; e < cnt; ++e) out[e] = static_cast<uint16_t>(o[e]);
      }
    } else {
      uint32_t* out = static_cast<uint32_t*>(a.out) + e0;
      if (cnt == 8 && (e0 & 3) == 0) {
        reinterpret_cast<u32x4*>(out)[0] = u32x4{o[0], o[1], o[2], o[3]};
        reinterpret_cast<u32x4*>(out)[1] = u32x4{o[4], o[5], o[6], o[7]};
      } else {
        for (int e = 0; e < cnt; ++e) out[e] = o[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Dequantize to the fragment-tiled bf16 layout of the prefill GEMM
// (tiled_unit in w4_internal.h; N % 32 == 0, K % 64 == 0, contiguous groups
// with G % 32 == 0 or a g_idx).  A workgroup owns one 32-row block and a
// range of 64-column K-steps.  Every (row, group) pair the range touches gets
// a 16-entry table of its bf16 values fp32(v) * s (the same values as the row
// dequantizers), so a nibble becomes one LDS read.  Thread t serves row
// rr = t % 32, K-step half h = (t / 32) % 2 and K-steps kq = t / 64 + 4 i: it
// loads the 16 code bytes of its 32 columns, looks up 32 values and writes
// four 16-byte units; the 64 lanes of a wave write 1 KB contiguously.
// ---------------------------------------------------------------------------
constexpr int kTiledRows = 32;

struct TiledPlan {
  int kt_per_block, blocks_k, groups;   // K-steps per workgroup, workgroups along K, table groups per row
  size_t lds;
};

__host__ __device__ inline int tiled_table_stride(int groups) {   // bytes per row: 32 per group, +4 against bank conflicts
  return groups * 32 + 4;
}

template <bool ASYM, bool GIDX>
__global__ __launch_bounds__(kDThreads) void dequantize_tiled_kernel(DequantArgs a, int kt_per_block, int groups) {
  extern __shared__ __attribute__((aligned(16))) uint8_t tsm[];
  const int K = static_cast<int>(a.K);
  const int KT = K / 64;
  const int NG = static_cast<int>(a.NG);
  const int G = static_cast<int>(a.G);
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kTiledRows;
  const int kt0 = blockIdx.y * kt_per_block;
  const int kt1 = min(KT, kt0 + kt_per_block);
  // groups of the table: all of them with a g_idx, else those the K range covers
  const int g_first = GIDX ? 0 : (64 * kt0) / G;
  const int stride = tiled_table_stride(groups);
  // with a g_idx: the table byte offset of each column's group, uint16 per
  // column of the range, after the value table
  uint16_t* gtab = reinterpret_cast<uint16_t*>(tsm + kTiledRows * stride);

  // 0. this thread's code words: K-steps kq + 4 i of the range, 16 bytes
  //    (32 columns) each, issued first so that the table work overlaps them
  const int rr = threadIdx.x % 32, h = (threadIdx.x / 32) % 2, kq = threadIdx.x / 64;
  const int64_t n = row0 + rr;
  const int64_t KB = a.K / 2;
  constexpr int kIt = 4;   // K-steps per thread and batch
  u32x4 cw[kIt];
  auto load_batch = [&](int ktb) {
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int kt = min(ktb + 4 * i, kt1 - 1);   // past the range: the last again, not stored
      cw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.codes + n * KB + 32 * kt + 16 * h));
    }
  };
  load_batch(kt0 + kq);

  // 1. tables: values, entry (row r, group g_first + gl, nibble u) at
  //    r * stride + gl * 32 + 2 u; group offsets of the range's columns
  for (int p = threadIdx.x; p < kTiledRows * groups; p += kDThreads) {
    const int r = p / groups, gl = p % groups;
    const int g = min(g_first + gl, NG - 1);
    const int64_t gi = (row0 + r) * a.NG + g;
    const float sc = a.scales[gi];
    const int z = ASYM ? static_cast<int>(zero_row(a.zeros, row0 + r, a.NG, a.zpk)[g]) : 8;
    uint32_t wv[8];
#pragma unroll
    for (int u = 0; u < 16; u += 2) {
      // value formed in integers (signed codes: (u ^ 8) - 8), then one fp32 multiply
      const float v0 = static_cast<float>((ASYM ? u : (u ^ 8)) - z) * sc;
      const float v1 = static_cast<float>((ASYM ? u + 1 : ((u + 1) ^ 8)) - z) * sc;
      wv[u / 2] = f32_to_bf16(v0) | (f32_to_bf16(v1) << 16);
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(tsm + r * stride + gl * 32);
#pragma unroll
    for (int q = 0; q < 8; ++q) dst[q] = wv[q];
  }
  if constexpr (GIDX) {
    const int ncols = 64 * (kt1 - kt0);
    for (int c = threadIdx.x; c < ncols; c += kDThreads)
      gtab[c] = static_cast<uint16_t>(min(max(a.g_idx[64 * kt0 + c], 0), NG - 1) * 32);
  }
  __syncthreads();

  // 2. lookups and tiled stores
  const uint8_t* trow = tsm + rr * stride;
  uint16_t* out = static_cast<uint16_t*>(a.out);
  for (int ktb = kt0 + kq; ktb < kt1; ktb += 4 * kIt) {
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int kt = ktb + 4 * i;
      if (kt >= kt1) break;
      const int c0 = 64 * kt + 32 * h;   // first of the thread's 32 columns
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // unit (ks, h): columns c0 + 8 ks .. + 7, code word ks
        uint32_t goff[8];
        if constexpr (GIDX) {
          const u32x4 gq = *reinterpret_cast<const u32x4*>(gtab + (c0 - 64 * kt0) + 8 * ks);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            goff[2 * e] = gq[e] & 0xFFFFu;
            goff[2 * e + 1] = gq[e] >> 16;
          }
        } else {
          const uint32_t go = static_cast<uint32_t>(c0 / G - g_first) * 32;
#pragma unroll
          for (int e = 0; e < 8; ++e) goff[e] = go;
        }
        const uint32_t d = cw[i][ks];
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t u0 = (d >> (4 * e)) & 15u, u1 = (d >> (4 * e + 4)) & 15u;
          const uint32_t lo = *reinterpret_cast<const uint16_t*>(trow + goff[e] + 2 * u0);
          const uint32_t hi = *reinterpret_cast<const uint16_t*>(trow + goff[e + 1] + 2 * u1);
          o[e / 2] = lo | (hi << 16);
        }
        const int64_t unit = ((static_cast<int64_t>(blockIdx.x) * KT + kt) * 4 + ks) * 64 + 32 * h + rr;
        // a plain store, not a streaming one: the GEMM reads the workspace
        // right after and finds it in the Infinity Cache (76.0 against
        // 78.3 us per prefill linear)
        *reinterpret_cast<u32x4*>(out + 8 * unit) = u32x4{o[0], o[1], o[2], o[3]};
      }
    }
    if (ktb + 4 * kIt < kt1) load_batch(ktb + 4 * kIt);
  }
}

TiledPlan tiled_plan(const DequantArgs& a) {
  TiledPlan p{};
  const int64_t KT = a.K / 64;
  const int64_t row_blocks = a.N / kTiledRows;
  // about 512 workgroups (two per CU), at least 4 K-steps each
  int64_t per = std::max<int64_t>(4, (KT * row_blocks + 511) / 512);
  per = std::min(per, KT);
  p.kt_per_block = static_cast<int>(per);
  p.blocks_k = static_cast<int>((KT + per - 1) / per);
  if (a.g_idx) {
    p.groups = static_cast<int>(a.NG);
  } else {
    // groups a range of `per` K-steps can touch (start anywhere)
    p.groups = static_cast<int>(std::min<int64_t>(a.NG, (64 * per + a.G - 1) / a.G + 1));
  }
  p.lds = static_cast<size_t>(kTiledRows) * tiled_table_stride(p.groups) + (a.g_idx ? 2 * 64 * per : 0);
  return p;
}

template <bool OUT_BF16, bool ASYM, int GIDX>
hipError_t launch_d3(const DequantArgs& a, hipStream_t s) {
  const int64_t nchunks = (a.K + 7) / 8;
  const int cb = static_cast<int>((nchunks + kDThreads - 1) / kDThreads);
  const dim3 grid(static_cast<uint32_t>(a.N * cb)), block(kDThreads);
  const size_t lds = GIDX == 1 ? static_cast<size_t>((a.NG * 5 + 15) / 16 * 16) : 0;
  dequantize_kernel<OUT_BF16, ASYM, GIDX><<<grid, block, lds, s>>>(a, cb);
  return hipGetLastError();
}

template <bool OUT_BF16, bool ASYM>
hipError_t launch_d2(const DequantArgs& a, hipStream_t s) {
  if (!a.g_idx) {
    if ((a.G & (a.G - 1)) == 0 && a.K >= 1024) {
      int lg = 0;
      while ((int64_t{1} << lg) < a.G) ++lg;
      dequantize_rows_kernel<OUT_BF16, ASYM><<<dim3(static_cast<uint32_t>(a.N)), dim3(kDThreads), 0, s>>>(a, lg);
      return hipGetLastError();
    }
    return launch_d3<OUT_BF16, ASYM, 0>(a, s);
  }
  if (a.K >= 512) {
    const int rows = act_rows<OUT_BF16>(a.NG);
    if (rows >= 4 && (a.N + rows - 1) / rows <= 65535) {
      const dim3 grid(static_cast<uint32_t>((a.K + 8 * kDThreads - 1) / (8 * kDThreads)),
                      static_cast<uint32_t>((a.N + rows - 1) / rows));
      const size_t lds = static_cast<size_t>(rows) * a.NG * 16 * act_entry_bytes<OUT_BF16>();
      dequantize_act_kernel<OUT_BF16, ASYM><<<grid, dim3(kDThreads), lds, s>>>(a, rows);
      return hipGetLastError();
    }
  }
  if (a.NG <= kDequantLdsGroups) return launch_d3<OUT_BF16, ASYM, 1>(a, s);
  return launch_d3<OUT_BF16, ASYM, 2>(a, s);
}

}  // namespace

hipError_t launch_quantize_pack(const QuantArgs& a, hipStream_t s) {
  if (a.w_bf16) return a.asym ? launch_q2<true, true>(a, s) : launch_q2<true, false>(a, s);
  return a.asym ? launch_q2<false, true>(a, s) : launch_q2<false, false>(a, s);
}

bool dequantize_tiled_ok(const DequantArgs& a) {
  if (!a.out_bf16 || a.N % 128 != 0 || a.K % 64 != 0 || a.N / kTiledRows > 65535) return false;
  if (!a.g_idx && a.G % 32 != 0) return false;
  return tiled_plan(a).lds <= 65536;
}

hipError_t launch_dequantize_tiled(const DequantArgs& a, hipStream_t s) {
  if (!dequantize_tiled_ok(a)) return hipErrorInvalidValue;
  const TiledPlan p = tiled_plan(a);
  const dim3 grid(static_cast<uint32_t>(a.N / kTiledRows), static_cast<uint32_t>(p.blocks_k));
  if (a.g_idx) {
    if (a.asym) dequantize_tiled_kernel<true, true><<<grid, dim3(kDThreads), p.lds, s>>>(a, p.kt_per_block, p.groups);
    else dequantize_tiled_kernel<false, true><<<grid, dim3(kDThreads), p.lds, s>>>(a, p.kt_per_block, p.groups);
  } else {
    if (a.asym) dequantize_tiled_kernel<true, false><<<grid, dim3(kDThreads), p.lds, s>>>(a, p.kt_per_block, p.groups);
    else dequantize_tiled_kernel<false, false><<<grid, dim3(kDThreads), p.lds, s>>>(a, p.kt_per_block, p.groups);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t s) {
  if (a.out_bf16) return a.asym ? launch_d2<true, true>(a, s) : launch_d2<true, false>(a, s);
  return a.asym ? launch_d2<false, true>(a, s) : launch_d2<false, false>(a, s);
}

}  // namespace w4
