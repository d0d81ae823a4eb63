// Batched decode on the matrix cores, one launch: y = x Wd^T + b for
// 4 < M <= 16 with contiguous groups (keras dense.py diff page:
// Dense._int4_call, the matmul with the dequantized kernel then the bias add;
// PaddleNLP quantization_linear.py page: weight_only_linear with group_size).
//
// v_mfma_f32_16x16x32_bf16 takes the activations as the 16-row A operand
// (rows m >= M repeat row M - 1 and are not stored) and 16 weight rows as the
// B operand, each nibble decoded to the bf16 value 128 + u.  The offset and
// the zero-point leave through the same matrix cores: one more MFMA per
// group multiplies the activations by the constant operand -(128 + z) (exact
// in bf16 for z <= 15) and seeds the group's accumulator, so that it ends as
// sum_k x_k (u_k - z) and the group's scale is one multiply-add per output.
//
// Workgroup = 4 waves on 64 weight rows (four 16-row blocks); wave w takes a
// quarter of K in pairs of 128-column batches and the four partial tiles are
// added in LDS in wave order.  Every global load instruction reads whole
// cache lines: code words as 8 rows x 128 bytes, activations as 4 rows x 256
// bytes; both pass through small wave-private LDS buffers into the MFMA
// operand layout (lane l: row l % 16, quarter q = l / 16 of the columns).
// Loaded in that layout directly, every instruction would touch 16 rows x 64
// bytes, and such loads run at about half the rate (measured with the
// arithmetic taken out).  Loads retire in order, so while a pair is computed
// the next pair's loads are in flight (8 KB of code words per wave); the pair
// index of a prefetch is clamped to the wave's last pair so that every round
// issues the same loads and the waits stay exact.  The scales (and
// zero-points) of the wave's rows and groups are read once, row-contiguous,
// into a wave-private LDS table before the loop: read per batch from global
// memory they would be 8 bytes from each of 16 rows per load instruction,
// which costs as much as the code words themselves.
#include "w4_device.h"
#include "w4_dot.h"
#include "w4_internal.h"
#include "w4_mfma.h"

namespace w4 {
namespace {

constexpr int kBWaves = 4;               // waves per workgroup, one quarter of K each
constexpr int kBRB = 4;                  // 16-row blocks per workgroup
constexpr int kBRows = 16 * kBRB;        // weight rows per workgroup
// table groups per row, at most: the tables (plus the activation buffers and
// the 12 KB reduction buffer) stay within 64 KB per workgroup
constexpr int kBMaxGroups = 32;          // scales only
constexpr int kBMaxGroupsZ = 16;         // scales and zero-points

// A wave's batches [bb, be) and groups [g_lo, g_lo + count).
struct BRange {
  int bb, be;
  int64_t g_lo, count;
};
__host__ __device__ inline BRange b_range(int w, int64_t K, int64_t G) {
  const int nb = static_cast<int>(K / 128);
  BRange r;
  r.bb = w * nb / kBWaves;
  r.be = (w + 1) * nb / kBWaves;
  r.g_lo = 128 * static_cast<int64_t>(r.bb) / G;
  r.count = r.bb < r.be ? (128 * static_cast<int64_t>(r.be) - 1) / G + 1 - r.g_lo : 0;
  return r;
}
// Table row stride in words: the largest group count of the four waves,
// made odd so that the 16 rows a load instruction reads fall on distinct banks.
__host__ __device__ inline int b_table_stride(int64_t K, int64_t G) {
  int64_t m = 1;
  for (int w = 0; w < kBWaves; ++w) {
    const int64_t c = b_range(w, K, G).count;
    m = c > m ? c : m;
  }
  return static_cast<int>(m | 1);
}

// A pair of batches (256 columns) of a wave's operands, loaded as whole
// cache lines: load j of the activations holds rows 4 (j % 4) + l / 16, batch
// j / 4, bytes 16 (l % 16); load i of the code words holds rows 16 (i / 2) +
// 8 (i % 2) + l / 8 of the workgroup, bytes 16 (l % 8) of the pair's 128.
struct BStage {
  u32x4 x[8];
  u32x4 cw[2 * kBRB];
};

// A wave's row pointers and lane offsets, computed once: lane l reads the
// activations of row min(l % 16, M - 1) and its quarter q = l / 16 of each
// row block's code words.  MFMA step s of a batch at column k0 sums, in lane
// quarter q, columns
//   k0 + 32 s + 8 q .. + 7   (U > 1: step s lies in one group), or
//   k0 + 32 q + 8 s .. + 7   (U = 1: the code word's own order).
// Offsets are 32-bit from the arrays' bases (the shape check keeps them
// below 2^31), so that every load takes a uniform base and one lane offset.
template <int U>
struct BRows {
  const uint8_t* xb;             // activations
  const uint8_t* cb;             // code words
  uint32_t x[4];                 // byte offset of activation row 4 s + l / 16 (at most M - 1) + 16 (l % 16)
  uint32_t c[2 * kBRB];          // byte offset of code row 8 i + l / 8 (at most N - 1) + 16 (l % 8)
  uint32_t gdiv;                 // G / 128 for U = 1

  __device__ __forceinline__ BRows(const LinearArgs& a, int64_t n0, int lane) {
    const int q = lane >> 4, r = lane & 15;
    const uint32_t K = static_cast<uint32_t>(a.K), N1 = static_cast<uint32_t>(a.N - 1);
    xb = reinterpret_cast<const uint8_t*>(a.x);
    cb = a.codes;
#pragma unroll
    for (int s = 0; s < 4; ++s) x[s] = static_cast<uint32_t>(min(4 * s + q, static_cast<int>(a.M) - 1)) * 2u * K + 16u * r;
#pragma unroll
    for (int i = 0; i < 2 * kBRB; ++i)
      c[i] = min(static_cast<uint32_t>(n0) + 8u * i + static_cast<uint32_t>(lane >> 3), N1) * (K / 2u) + 16u * (lane & 7);
    gdiv = static_cast<uint32_t>(a.G / 128);
  }
  // first group of batch b
  __device__ __forceinline__ uint32_t group(uint32_t b) const { return U > 1 ? U * b : b / gdiv; }
};

// the loads of batch pair p (batches 2 p, 2 p + 1)
template <int U>
__device__ __forceinline__ void b_issue(const BRows<U>& R, uint32_t p, BStage& st) {
#pragma unroll
  for (int j = 0; j < 8; ++j) st.x[j] = *reinterpret_cast<const u32x4*>(R.xb + (R.x[j & 3] + 512u * p + 256u * (j >> 2)));
#pragma unroll
  for (int i = 0; i < 2 * kBRB; ++i)   // code words are read once: non-temporal
    st.cw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(R.cb + (R.c[i] + 128u * p)));
  __builtin_amdgcn_sched_barrier(0);
}

// The wave's scale (and zero-point) table: row r (0 .. 63) of the workgroup,
// group g_lo + c at word r * S + c.  Pass p stores rows p * (64 / count) +
// l / count, column l % count of lane l; row indices past 63 repeat row 63.
template <int ZP>
__device__ __forceinline__ void b_table(const LinearArgs& a, int64_t n0, const BRange& br, int S, int lane,
                                        float* stab, uint32_t* ztab) {
  const int cnt = static_cast<int>(br.count);
  const int per = kWave / cnt;                      // rows per pass (cnt <= 32: at least 2)
  const int lr = lane / cnt, c = lane - lr * cnt;
  float sv[kWave / 2];
  uint32_t zv[kWave / 2];
  const uint32_t NG = static_cast<uint32_t>(a.NG), N1 = static_cast<uint32_t>(a.N - 1);
  const uint32_t g = static_cast<uint32_t>(br.g_lo) + static_cast<uint32_t>(c);
#pragma unroll
  for (int p = 0; p < kWave / 2; ++p) {
    const uint32_t r = static_cast<uint32_t>(min(p * per + lr, kBRows - 1));
    const uint32_t n = min(static_cast<uint32_t>(n0) + r, N1);
    sv[p] = *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.scales) + 4u * (n * NG + g));
    if constexpr (ZP == 1) zv[p] = a.zeros[n * NG + g];
    if constexpr (ZP == 2) zv[p] = a.zeros[n * ((NG + 1u) >> 1) + (g >> 1)];
  }
#pragma unroll
  for (int p = 0; p < kWave / 2; ++p) {
    const int r = min(p * per + lr, kBRows - 1);
    stab[r * S + c] = sv[p];
    if constexpr (ZP != 0) ztab[r * S + c] = zero_of<ZP == 2>(zv[p], static_cast<uint32_t>(br.g_lo + c));
  }
}

// The wave's LDS buffers.  Activations: row m (256 bytes of a batch) at
// m * kBXRow; code words: row r of a row block (128 bytes of a pair) at
// r * kBCRow.  The 16-byte pads put the 16 rows a read pass touches on
// distinct banks.
constexpr int kBXRow = 272;
constexpr int kBXBytes = 16 * kBXRow;
constexpr int kBCRow = 144;
constexpr int kBCBytes = 16 * kBCRow;

// Batch b = 2 p + j of the pair's operands in st.
template <int ZP, int U>
__device__ __forceinline__ void b_batch(const BRows<U>& R, uint32_t b, int j, const BStage& st,
                                        const uint32_t (&dw)[kBRB][2][4], uint32_t mask, const float* stab,
                                        const uint32_t* ztab, int S, uint32_t g_lo, int lane, uint8_t* xl,
                                        float (&out)[kBRB][4]) {
  constexpr bool TR = U > 1;
  constexpr int SPU = 4 / U;   // MFMA steps per group
  const int q = lane >> 4, m = lane & 15;
  // activations -> LDS (row 4 s + q, chunk m), then the operand layout: lane
  // (m, q) of step s takes 16 bytes of row m at column 32 s + 8 q (TR) or 32 q + 8 s
#pragma unroll
  for (int s = 0; s < 4; ++s) *reinterpret_cast<u32x4*>(xl + (4 * s + q) * kBXRow + 16 * m) = st.x[4 * j + s];
  u32x4 xr[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) xr[s] = *reinterpret_cast<const u32x4*>(xl + m * kBXRow + (TR ? 64 * s + 16 * q : 64 * q + 16 * s));
  bf16x8_t xa[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t in[4] = {xr[s][0], xr[s][1], xr[s][2], xr[s][3]};
    uint32_t xp[4];
    pair_x(in, xp);
    xa[s] = __builtin_bit_cast(bf16x8_t, u32x4{xp[0], xp[1], xp[2], xp[3]});
  }
  const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  // signed codes: every row's offset is 128 + 8, one seed per group for all blocks
  f32x4_t seed[U];
  if constexpr (ZP == 0) {
    const bf16x8_t c136 = __builtin_bit_cast(bf16x8_t, u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u});
#pragma unroll
    for (int u = 0; u < U; ++u) {
      seed[u] = zero4;
#pragma unroll
      for (int s = u * SPU; s < (u + 1) * SPU; ++s)
        seed[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[s], c136, seed[u], 0, 0, 0);
    }
  }
  const int c0 = static_cast<int>(R.group(b) - g_lo);   // table column of the batch's first group
  const int n = lane & 15;
#pragma unroll
  for (int rb = 0; rb < kBRB; ++rb) {
    uint32_t d[4] = {dw[rb][j][0], dw[rb][j][1], dw[rb][j][2], dw[rb][j][3]};
    if constexpr (ZP == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] ^= 0x88888888u;   // signed q -> q + 8
    }
    const int trow = (16 * rb + n) * S + c0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4_t acc;
      if constexpr (ZP == 0) {
        acc = seed[u];
      } else {
        // bf16 -(128 + z): sign, the exponent of 128, z in the low mantissa bits
        const uint32_t h = 0xC300u | ztab[trow + u];
        const uint32_t hz = h | (h << 16);
        const bf16x8_t cz = __builtin_bit_cast(bf16x8_t, u32x4{hz, hz, hz, hz});
        acc = zero4;
#pragma unroll
        for (int s = u * SPU; s < (u + 1) * SPU; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[s], cz, acc, 0, 0, 0);
      }
#pragma unroll
      for (int s = u * SPU; s < (u + 1) * SPU; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[s], decode_word(d[s], mask), acc, 0, 0, 0);
      const float sc = stab[trow + u];
#pragma unroll
      for (int t = 0; t < 4; ++t) out[rb][t] = __builtin_fmaf(sc, acc[t], out[rb][t]);
    }
  }
}

// Batch pair p: the code words of each row block pass through LDS (rows
// 8 (i % 2) + l / 8, chunk l % 8) into the operand layout, then the two
// batches.  Lane (n, q) of batch j reads row n: for U = 1 the 16 bytes of
// chunk 4 j + q (MFMA step s sums columns 32 q + 8 s .. of the batch); for
// U > 1 the four dwords at columns 32 s + 8 q (step s sums one group's 32
// columns), which the reads take straight from the rows, so no cross-lane
// transpose is needed.
template <int ZP, int U>
__device__ __forceinline__ void b_compute(const BRows<U>& R, uint32_t p, const BStage& st, uint32_t mask,
                                          const float* stab, const uint32_t* ztab, int S, uint32_t g_lo, int lane,
                                          uint8_t* xl, uint8_t* cl, float (&out)[kBRB][4]) {
  const int q = lane >> 4, n = lane & 15;
  uint32_t dw[kBRB][2][4];
#pragma unroll
  for (int rb = 0; rb < kBRB; ++rb) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<u32x4*>(cl + (8 * h + (lane >> 3)) * kBCRow + 16 * (lane & 7)) = st.cw[2 * rb + h];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (U > 1) {
        const uint32_t* crow = reinterpret_cast<const uint32_t*>(cl + n * kBCRow + 64 * j + 4 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) dw[rb][j][i] = crow[4 * i];
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(cl + n * kBCRow + 16 * (4 * j + q));
#pragma unroll
        for (int i = 0; i < 4; ++i) dw[rb][j][i] = v[i];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) b_batch<ZP, U>(R, 2 * p + j, j, st, dw, mask, stab, ztab, S, g_lo, lane, xl, out);
}

// Dynamic LDS: per wave an activation buffer (kBXBytes) and a code buffer
// (kBCBytes), then per wave a scale table [64][S] floats and (zero-points) a
// zero table [64][S] words.
template <int ZP, int U>
__global__ __launch_bounds__(kBWaves * kWave, 2) void batched_kernel(LinearArgs a, int S) {
  extern __shared__ __attribute__((aligned(16))) uint8_t btab[];
  __shared__ float red[kBWaves - 1][kBRB * 4][kWave];
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kBRows;   // rows past N: computed, not stored
  const BRange br = b_range(w, a.K, a.G);
  uint8_t* xl = btab + w * (kBXBytes + kBCBytes);
  uint8_t* cl = xl + kBXBytes;
  float* stab = reinterpret_cast<float*>(btab + kBWaves * (kBXBytes + kBCBytes)) + (ZP ? 2 : 1) * w * kBRows * S;
  uint32_t* ztab = reinterpret_cast<uint32_t*>(stab + kBRows * S);
  const uint32_t mask = nibble_mask();
  float out[kBRB][4];
#pragma unroll
  for (int rb = 0; rb < kBRB; ++rb)
#pragma unroll
    for (int t = 0; t < 4; ++t) out[rb][t] = 0.0f;

  if (br.bb < br.be) {
    const BRows<U> R(a, n0, lane);
    const uint32_t p0 = static_cast<uint32_t>(br.bb) / 2, pl = static_cast<uint32_t>(br.be - 1) / 2;
    const uint32_t g_lo = static_cast<uint32_t>(br.g_lo);
    BStage st[2];
    b_issue<U>(R, p0, st[0]);
    b_table<ZP>(a, n0, br, S, lane, stab, ztab);   // wave-private: the wave's own LDS writes precede its reads
    // whole rounds of two pairs while a pair follows them, with no exit
    // inside the loop body (an exit would leave stage loads pending on a path
    // back to the loop head, and the wait there would cover every load in
    // flight); the last one or two pairs after the loop, so that no pair is
    // loaded twice
    uint32_t p = p0;
    for (; p + 2 <= pl; p += 2) {
      b_issue<U>(R, p + 1, st[1]);
      b_compute<ZP, U>(R, p, st[0], mask, stab, ztab, S, g_lo, lane, xl, cl, out);
      b_issue<U>(R, p + 2, st[0]);
      b_compute<ZP, U>(R, p + 1, st[1], mask, stab, ztab, S, g_lo, lane, xl, cl, out);
    }
    if (p + 1 <= pl) {
      b_issue<U>(R, p + 1, st[1]);
      b_compute<ZP, U>(R, p, st[0], mask, stab, ztab, S, g_lo, lane, xl, cl, out);
      b_compute<ZP, U>(R, p + 1, st[1], mask, stab, ztab, S, g_lo, lane, xl, cl, out);
    } else {
      b_compute<ZP, U>(R, p, st[0], mask, stab, ztab, S, g_lo, lane, xl, cl, out);   // already in st[0]
    }
  }

  // the K quarters' tiles meet in LDS; wave 0 adds them in wave order
  if (w > 0) {
#pragma unroll
    for (int rb = 0; rb < kBRB; ++rb)
#pragma unroll
      for (int t = 0; t < 4; ++t) red[w - 1][4 * rb + t][lane] = out[rb][t];
  }
  __syncthreads();
  if (w > 0) return;
  const int n = lane & 15, q = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < kBRB; ++rb) {
    const int64_t row = n0 + 16 * rb + n;
    if (row >= a.N) continue;
    const float bias = a.bias ? bf16_to_f32(a.bias[row]) : 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float v = out[rb][t];
#pragma unroll
      for (int ww = 0; ww < kBWaves - 1; ++ww) v += red[ww][4 * rb + t][lane];
      const int m = 4 * q + t;                      // output row of lane (n, q), slot t
      if (m < a.M) a.y[static_cast<int64_t>(m) * a.N + row] = static_cast<uint16_t>(f32_to_bf16(v + bias));
    }
  }
}

size_t b_lds_bytes(int64_t K, int64_t G, bool asym) {
  return static_cast<size_t>(kBWaves) * (kBXBytes + kBCBytes + kBRows * b_table_stride(K, G) * 4 * (asym ? 2 : 1));
}

template <int ZP>
hipError_t launch_batched2(const LinearArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>((a.N + kBRows - 1) / kBRows)), block(kBWaves * kWave);
  const int S = b_table_stride(a.K, a.G);
  const size_t lds = b_lds_bytes(a.K, a.G, ZP != 0);
  if (a.G == 32) batched_kernel<ZP, 4><<<grid, block, lds, s>>>(a, S);
  else if (a.G == 64) batched_kernel<ZP, 2><<<grid, block, lds, s>>>(a, S);
  else batched_kernel<ZP, 1><<<grid, block, lds, s>>>(a, S);
  return hipGetLastError();
}

}  // namespace

// Contiguous groups of 32, 64 or a multiple of 128 columns, K a multiple of
// 1024 (every wave's quarter of K is whole batch pairs), 4 < M <= 16, at most
// 32 groups (16 with zero-points) in a quarter of K (the table), and codes
// and activations whose byte offsets fit in 31 bits.
bool batched_shape_ok(int64_t N, int64_t M, int64_t K, int64_t G, bool has_g_idx, bool asym) {
  if (has_g_idx || K % 1024 != 0 || M <= 4 || M > 16 || !(G == 32 || G == 64 || G % 128 == 0)) return false;
  const int64_t lim = int64_t{1} << 31;   // 32-bit offsets
  if (N * (K / 2) >= lim || M * K * 2 >= lim || N * ((K + G - 1) / G) * 4 >= lim) return false;
  for (int w = 0; w < kBWaves; ++w)
    if (b_range(w, K, G).count > (asym ? kBMaxGroupsZ : kBMaxGroups)) return false;
  return true;
}
bool batched_ok(const LinearArgs& a) { return batched_shape_ok(a.N, a.M, a.K, a.G, a.g_idx != nullptr, a.asym != 0); }

hipError_t launch_batched(const LinearArgs& a, hipStream_t s) {
  if (!a.asym) return launch_batched2<0>(a, s);
  return a.zpk ? launch_batched2<2>(a, s) : launch_batched2<1>(a, s);
}

}  // namespace w4
