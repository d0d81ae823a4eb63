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
__global__ __launch_bounds__(kQThreads) void quantize_pack_kernel(QuantArgs a) {
  extern __shared__ uint32_t lds[];
  const int NG = static_cast<int>(a.NG);
  const int K = static_cast<int>(a.K);
  const int G = static_cast<int>(a.G);
  const int64_t n = blockIdx.x;
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
      if constexpr (ASYM) zt[g] = a.zeros[n * a.NG + g];
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
  const uint8_t* zrow = ASYM ? a.zeros + n * a.NG : nullptr;
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
  return a.g_idx ? launch_q3<BF16, ASYM, true>(a, s) : launch_q3<BF16, ASYM, false>(a, s);
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
  if (!a.g_idx) return launch_d3<OUT_BF16, ASYM, 0>(a, s);
  if (a.NG <= kDequantLdsGroups) return launch_d3<OUT_BF16, ASYM, 1>(a, s);
  return launch_d3<OUT_BF16, ASYM, 2>(a, s);
}

}  // namespace

hipError_t launch_quantize_pack(const QuantArgs& a, hipStream_t s) {
  if (a.w_bf16) return a.asym ? launch_q2<true, true>(a, s) : launch_q2<true, false>(a, s);
  return a.asym ? launch_q2<false, true>(a, s) : launch_q2<false, false>(a, s);
}

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t s) {
  if (a.out_bf16) return a.asym ? launch_d2<true, true>(a, s) : launch_d2<true, false>(a, s);
  return a.asym ? launch_d2<false, true>(a, s) : launch_d2<false, false>(a, s);
}

}  // namespace w4
