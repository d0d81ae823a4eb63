// Storage formats next to the packed layout:
//
// Q4_0 blocks (Modular MAX quantization.py page: QuantizationEncoding,
// Q4_0 = 32 weights per block in 2 + 16 bytes, the scale d then 4-bit codes;
// the page fixes nothing more, so the rest is this library's reading).
// A block is the fp16 scale d (little-endian) followed by 16 bytes; byte i
// holds code q[i] + 8 in its low nibble and q[i + 16] + 8 in its high nibble;
// a weight reads as (q - 8) * d.  Quantization is the
// signed absmax rule of the packed format taken against the stored scale:
// d = fp16(fp32(amax / 7)), q = clamp(rint(fp32(w / d)), -7, 7), all codes 0
// when d is 0.
//
// The blocks of an [N, K] weight (K a multiple of 32) form one flat array:
// block g covers weights 32 g .. 32 g + 31 and bytes 18 g .. 18 g + 17.  The
// quantizer gives a lane one block; a wave's 64 blocks are 1152 contiguous,
// 16-byte aligned bytes, written through LDS as 72 coalesced 16-byte chunks.
// The dequantizer reads a wave's 128 blocks (2304 bytes) the same way.
//
// Packed zero-points: two per byte along the row, group 2j in the low nibble
// (the codes' order), an odd group count leaving the last high nibble 0.

#include "w4_device.h"
#include "w4_internal.h"

#include <algorithm>

namespace w4 {
namespace {

constexpr int kFThreads = 256;
constexpr int kQ4Block = 32;
constexpr int kQ4Bytes = 18;
constexpr int kQ4WaveBytes = kWave * kQ4Bytes;          // 1152 = 72 chunks of 16 bytes
constexpr int kQ4WaveChunks = kQ4WaveBytes / 16;
constexpr int kQ4DeqBlocks = 128;                       // blocks per wave when dequantizing

template <bool BF16>
__global__ __launch_bounds__(kFThreads) void q4_0_quantize_kernel(const void* __restrict__ w, int64_t nblocks,
                                                                   uint8_t* __restrict__ out) {
  // The wave's 64 blocks are one contiguous run of weights: they are read
  // with coalesced 16-byte loads (lane l of load c takes chunk 64 c + l of the
  // run, read once: non-temporal) into LDS rows of BB + 16 bytes (the padding
  // keeps each lane's row reads free of bank conflicts), then each lane reads
  // its own block.
  constexpr int BB = BF16 ? 64 : 128;   // input bytes per block
  constexpr int PB = BB + 16;
  constexpr int NI = BB / 16;           // 16-byte chunks per block
  __shared__ __attribute__((aligned(16))) uint8_t inb[kFThreads / kWave][kWave * PB];
  __shared__ __attribute__((aligned(16))) uint8_t stage[kFThreads / kWave][kQ4WaveBytes];
  const int lane = lane_id();
  const int wv = threadIdx.x >> 6;
  const int64_t g0 = (static_cast<int64_t>(blockIdx.x) * kFThreads) + kWave * wv;   // the wave's first block
  const int64_t g = g0 + lane;
  // blocks of this wave that exist (<= 0 for the trailing waves of the last
  // workgroup, which load nothing and store nothing but reach the barriers)
  const int64_t nvalid = min(static_cast<int64_t>(kWave), nblocks - g0);
  if (nvalid > 0) {
    const uint8_t* src = static_cast<const uint8_t*>(w) + g0 * BB;
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      const int i = min(kWave * c + lane, static_cast<int>(nvalid) * NI - 1);   // clamped: in bounds
      const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + i);
      *reinterpret_cast<u32x4*>(&inb[wv][(i / NI) * PB + (i % NI) * 16]) = q;
    }
  }
  __syncthreads();
  float v[kQ4Block];
  if constexpr (BF16) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(&inb[wv][lane * PB + 16 * c]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * c + 2 * i] = __uint_as_float(q[i] << 16);
        v[8 * c + 2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(&inb[wv][lane * PB + 16 * c]);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * c + i] = __uint_as_float(q[i]);
    }
  }

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kQ4Block; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const _Float16 d16 = static_cast<_Float16>(div_const<7>(amax));      // round to nearest even
  const float d = static_cast<float>(d16);

  // codes: rint(w / d) through the reciprocal with the exact redo near
  // half-integers (|w / d| <= 10.5 even for subnormal d), clamped to [-7, 7]
  float qf[kQ4Block];
  if (d != 0.0f) {
    bool redo = false;
#pragma unroll
    for (int c = 0; c < 4; ++c) redo |= quant8_fast(&v[8 * c], d, &qf[8 * c]);
    if (redo) {
#pragma unroll
      for (int c = 0; c < 4; ++c) quant8_redo(&v[8 * c], d, &qf[8 * c]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kQ4Block; ++i) qf[i] = 0.0f;
  }
  uint32_t word[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      lo = __builtin_amdgcn_cvt_pk_u8_f32(fminf(fmaxf(qf[4 * k + t], -7.0f), 7.0f) + 8.0f, t, lo);
      hi = __builtin_amdgcn_cvt_pk_u8_f32(fminf(fmaxf(qf[16 + 4 * k + t], -7.0f), 7.0f) + 8.0f, t, hi);
    }
    word[k] = lo | (hi << 4);
  }

  // the wave's blocks through LDS (2-byte granules: a block starts at an even
  // offset), then 72 chunks of 16 bytes
  uint16_t* st = reinterpret_cast<uint16_t*>(stage[wv] + kQ4Bytes * lane);
  if (g < nblocks) {
    st[0] = __builtin_bit_cast(uint16_t, d16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      st[1 + 2 * k] = static_cast<uint16_t>(word[k]);
      st[2 + 2 * k] = static_cast<uint16_t>(word[k] >> 16);
    }
  }
  __syncthreads();                      // every wave reaches this point
  uint8_t* dst = out + g0 * kQ4Bytes;
  if (nvalid == kWave) {
    const u32x4* sv = reinterpret_cast<const u32x4*>(stage[wv]);
    __builtin_nontemporal_store(sv[lane], reinterpret_cast<u32x4*>(dst) + lane);
    if (lane < kQ4WaveChunks - kWave)
      __builtin_nontemporal_store(sv[kWave + lane], reinterpret_cast<u32x4*>(dst) + kWave + lane);
  } else {
    const uint16_t* sv = reinterpret_cast<const uint16_t*>(stage[wv]);
    uint16_t* d2 = reinterpret_cast<uint16_t*>(dst);
    for (int i = lane; i < nvalid * (kQ4Bytes / 2); i += kWave) d2[i] = sv[i];
  }
}

// Dequantize: a wave takes 128 consecutive blocks (2304 bytes, 16-byte
// aligned), reads them with coalesced loads into LDS, then decodes them in
// rounds: in each round a lane turns WPL consecutive weights of one block (8
// for bf16, 4 for fp32 output: 16 bytes) into one store, so a round's stores
// are one contiguous run of 1 KB.
template <bool OUT_BF16>
__global__ __launch_bounds__(kFThreads) void q4_0_dequantize_kernel(const uint8_t* __restrict__ blocks,
                                                                     int64_t nblocks, void* __restrict__ out) {
  constexpr int kWPL = OUT_BF16 ? 8 : 4;                 // weights per lane and round
  constexpr int kLPB = kQ4Block / kWPL;                  // lanes per block
  constexpr int kBPR = kWave / kLPB;                     // blocks per round
  constexpr int kRounds = kQ4DeqBlocks / kBPR;
  constexpr int kChunks = kQ4DeqBlocks * kQ4Bytes / 16;  // 144
  __shared__ __attribute__((aligned(16))) uint8_t stage[kFThreads / kWave][kQ4DeqBlocks * kQ4Bytes];
  const int lane = lane_id();
  const int wv = threadIdx.x >> 6;
  const int64_t g0 = (static_cast<int64_t>(blockIdx.x) * (kFThreads / kWave) + wv) * kQ4DeqBlocks;
  // blocks of this wave that exist (<= 0 for the trailing waves of the last
  // workgroup, which load and store nothing but reach the barrier)
  const int64_t nvalid = min(static_cast<int64_t>(kQ4DeqBlocks), nblocks - g0);
  const uint8_t* src = blocks + g0 * kQ4Bytes;
  if (nvalid == kQ4DeqBlocks) {
#pragma unroll
    for (int i = 0; i < (kChunks + kWave - 1) / kWave; ++i) {
      const int c = lane + kWave * i;
      if (c < kChunks)
        reinterpret_cast<u32x4*>(stage[wv])[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + c);
    }
  } else if (nvalid > 0) {
    uint16_t* sv = reinterpret_cast<uint16_t*>(stage[wv]);
    const uint16_t* s2 = reinterpret_cast<const uint16_t*>(src);
    for (int i = lane; i < nvalid * (kQ4Bytes / 2); i += kWave) sv[i] = s2[i];
  }
  __syncthreads();                      // every wave reaches this point
  const int i0 = kWPL * (lane % kLPB);  // first weight of the lane in its block
  // code bytes (i0 mod 16) .. + WPL - 1 of the block: low nibbles for the
  // first 16 weights, high nibbles for the last 16
  const int b0 = i0 & 15;
  const int sh = i0 < 16 ? 0 : 4;
#pragma unroll 4
  for (int r = 0; r < kRounds; ++r) {
    const int bl = kBPR * r + lane / kLPB;   // block of the wave
    if (bl >= nvalid) break;
    const uint16_t* st = reinterpret_cast<const uint16_t*>(stage[wv] + kQ4Bytes * bl);
    const float d = static_cast<float>(__builtin_bit_cast(_Float16, st[0]));
    float v[kWPL];
#pragma unroll
    for (int h = 0; h < kWPL / 2; ++h) {
      const uint32_t two = st[1 + (b0 >> 1) + h];        // bytes b0 + 2h, b0 + 2h + 1 (b0 is even)
      v[2 * h] = static_cast<float>(static_cast<int>((two >> sh) & 15u) - 8) * d;
      v[2 * h + 1] = static_cast<float>(static_cast<int>((two >> (8 + sh)) & 15u) - 8) * d;
    }
    const int64_t g = g0 + bl;
    if constexpr (OUT_BF16) {
      u32x4 q;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2_t p = {static_cast<__bf16>(v[2 * i]), static_cast<__bf16>(v[2 * i + 1])};
        q[i] = __builtin_bit_cast(uint32_t, p);
      }
      __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + g * kQ4Block + i0));
    } else {
      __builtin_nontemporal_store(f32x4_t{v[0], v[1], v[2], v[3]},
                                  reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + g * kQ4Block + i0));
    }
  }
}

// packed[n, j] = z[n, 2j] | z[n, 2j + 1] << 4  (0 past the last group)
__global__ __launch_bounds__(kFThreads) void pack_zeros_kernel(const uint8_t* __restrict__ z, int64_t N, int64_t NG,
                                                               uint8_t* __restrict__ packed) {
  const int64_t NB = (NG + 1) / 2;
  const int64_t total = N * NB;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kFThreads + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * kFThreads) {
    const int64_t n = i / NB, j = i - n * NB;
    const uint32_t lo = z[n * NG + 2 * j] & 15u;
    const uint32_t hi = 2 * j + 1 < NG ? (z[n * NG + 2 * j + 1] & 15u) : 0u;
    packed[i] = static_cast<uint8_t>(lo | (hi << 4));
  }
}

__global__ __launch_bounds__(kFThreads) void unpack_zeros_kernel(const uint8_t* __restrict__ packed, int64_t N,
                                                                 int64_t NG, uint8_t* __restrict__ z) {
  const int64_t NB = (NG + 1) / 2;
  const int64_t total = N * NG;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kFThreads + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * kFThreads) {
    const int64_t n = i / NG, g = i - n * NG;
    z[i] = static_cast<uint8_t>((packed[n * NB + g / 2] >> (4 * (g & 1))) & 15u);
  }
}

// Even NG: rows pack to whole bytes, so the tables are flat arrays with
// packed[i] = z[2i] | z[2i+1] << 4; a thread takes 16 zero-points (one
// 16-byte load, one 8-byte store) and the last partial piece goes bytewise.
__global__ __launch_bounds__(kFThreads) void pack_zeros_flat_kernel(const uint8_t* __restrict__ z, int64_t nout,
                                                                    uint8_t* __restrict__ packed) {
  const int64_t full = nout / 8;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kFThreads + threadIdx.x; i <= full;
       i += static_cast<int64_t>(gridDim.x) * kFThreads) {
    if (i < full) {
      const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(z) + i);
      uint32_t o[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t a = q[2 * h] & 0x0F0F0F0Fu, b = q[2 * h + 1] & 0x0F0F0F0Fu;
        // bytes (a0 a1 a2 a3) -> nibble pairs a0|a1<<4, a2|a3<<4 in the low half, b likewise in the high half
        const uint32_t pa = (a | (a >> 4)) & 0x00FF00FFu;      // a0|a1<<4 at byte 0, a2|a3<<4 at byte 2
        const uint32_t pb = (b | (b >> 4)) & 0x00FF00FFu;
        o[h] = (pa & 0xFFu) | ((pa >> 8) & 0xFF00u) | ((pb & 0xFFu) << 16) | ((pb >> 8) & 0xFF00u) << 16;
      }
      *reinterpret_cast<u32x2*>(packed + 8 * i) = u32x2{o[0], o[1]};
    } else {
      for (int64_t j = 8 * full; j < nout; ++j) packed[j] = static_cast<uint8_t>((z[2 * j] & 15u) | ((z[2 * j + 1] & 15u) << 4));
    }
  }
}

__global__ __launch_bounds__(kFThreads) void unpack_zeros_flat_kernel(const uint8_t* __restrict__ packed, int64_t nin,
                                                                      uint8_t* __restrict__ z) {
  const int64_t full = nin / 8;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kFThreads + threadIdx.x; i <= full;
       i += static_cast<int64_t>(gridDim.x) * kFThreads) {
    if (i < full) {
      const u32x2 p = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(packed) + i);
      u32x4 q;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w = p[h];
        // byte k of w -> bytes 2k (low nibble) and 2k+1 (high nibble)
        const uint32_t lo = (w & 0xFFu) | ((w & 0xFF00u) << 8);            // bytes 0, 1 of w at 0 and 2
        const uint32_t hi = ((w >> 16) & 0xFFu) | ((w >> 8) & 0xFF0000u);  // bytes 2, 3 of w at 0 and 2
        q[2 * h] = (lo & 0x000F000Fu) | ((lo & 0x00F000F0u) << 4);
        q[2 * h + 1] = (hi & 0x000F000Fu) | ((hi & 0x00F000F0u) << 4);
      }
      __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(z) + i);
    } else {
      for (int64_t j = 8 * full; j < nin; ++j) {
        z[2 * j] = packed[j] & 15u;
        z[2 * j + 1] = packed[j] >> 4;
      }
    }
  }
}

uint32_t grid_for(int64_t total) {
  return static_cast<uint32_t>(std::min<int64_t>((total + kFThreads - 1) / kFThreads, int64_t(1) << 20));
}

}  // namespace

hipError_t launch_q4_0_quantize(const void* w, bool bf16, int64_t N, int64_t K, uint8_t* blocks, hipStream_t s) {
  const int64_t nb = N * (K / kQ4Block);
  const dim3 grid(static_cast<uint32_t>((nb + kFThreads - 1) / kFThreads));
  if (bf16) q4_0_quantize_kernel<true><<<grid, dim3(kFThreads), 0, s>>>(w, nb, blocks);
  else q4_0_quantize_kernel<false><<<grid, dim3(kFThreads), 0, s>>>(w, nb, blocks);
  return hipGetLastError();
}

hipError_t launch_q4_0_dequantize(const uint8_t* blocks, int64_t N, int64_t K, void* out, bool bf16, hipStream_t s) {
  const int64_t nb = N * (K / kQ4Block);
  const int64_t per_wg = (kFThreads / kWave) * kQ4DeqBlocks;       // blocks per workgroup
  const dim3 grid(static_cast<uint32_t>((nb + per_wg - 1) / per_wg));
  if (bf16) q4_0_dequantize_kernel<true><<<grid, dim3(kFThreads), 0, s>>>(blocks, nb, out);
  else q4_0_dequantize_kernel<false><<<grid, dim3(kFThreads), 0, s>>>(blocks, nb, out);
  return hipGetLastError();
}

bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

hipError_t launch_pack_zeros(const uint8_t* z, int64_t N, int64_t NG, uint8_t* packed, hipStream_t s) {
  if (NG % 2 == 0 && aligned_to(z, 16) && aligned_to(packed, 8)) {
    const int64_t nout = N * NG / 2;
    pack_zeros_flat_kernel<<<dim3(grid_for(nout / 8 + 1)), dim3(kFThreads), 0, s>>>(z, nout, packed);
    return hipGetLastError();
  }
  pack_zeros_kernel<<<dim3(grid_for(N * ((NG + 1) / 2))), dim3(kFThreads), 0, s>>>(z, N, NG, packed);
  return hipGetLastError();
}

hipError_t launch_unpack_zeros(const uint8_t* packed, int64_t N, int64_t NG, uint8_t* z, hipStream_t s) {
  if (NG % 2 == 0 && aligned_to(z, 16) && aligned_to(packed, 8)) {
    const int64_t nin = N * NG / 2;
    unpack_zeros_flat_kernel<<<dim3(grid_for(nin / 8 + 1)), dim3(kFThreads), 0, s>>>(packed, nin, z);
    return hipGetLastError();
  }
  unpack_zeros_kernel<<<dim3(grid_for(N * NG)), dim3(kFThreads), 0, s>>>(packed, N, NG, z);
  return hipGetLastError();
}

}  // namespace w4
