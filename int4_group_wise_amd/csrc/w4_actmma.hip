// Act-order decode GEMV on the matrix cores, M = 1: y = x Wd^T + b when each
// column k has its own group g_idx[k] (keras dense.py diff page:
// Dense._int4_call and dequantize_with_sz_map with g_idx; MAX
// graph/quantization.py page: QuantizationConfig.desc_act).
//
// With act-order the columns of a group are scattered over the row, so a
// per-weight scale would need a gather per weight.  Instead the groups become
// the rows of the MFMA A operand: A[g][k] = x_k if g_idx[k] = g, else 0, so
// that v_mfma_f32_16x16x32_bf16 against the decoded weights (B, nibbles as
// 128 + u) gives C[g][n] = sum over the columns k of group g of x_k (128 + u).
// One more MFMA against an all-ones B gives each group's activation sum X_g,
// and the result is y[n] = sum_g s[n][g] (C[g][n] - (128 + z[n][g]) X_g): the
// scales and zero-points are read once per (row, group), at the end, from
// their rows.  A is built per 128-column batch in a wave-private LDS buffer
// (32 group rows x 128 columns, zero except one entry per column): each lane
// clears the two entries it wrote for the previous batch and writes its two
// columns' activations into their groups' rows, at the positions that make an
// aligned 16-byte read return the MFMA operand.
//
// Workgroup = 4 waves on 32 weight rows (two 16-row blocks), each wave a
// quarter of K in pairs of batches, as in the batched decode: code words are
// loaded as whole cache lines (8 rows x 128 bytes per instruction) and pass
// through a small LDS buffer into the operand layout; up to four pairs are in
// flight per wave (all of a 4096-column row's quarter); the waves' partial
// sums meet in LDS in wave order.
#include "w4_device.h"
#include "w4_dot.h"
#include "w4_internal.h"
#include "w4_mfma.h"

namespace w4 {
namespace {

constexpr int kAWaves = 4;                 // waves per workgroup, one quarter of K each
constexpr int kARB = 2;                    // 16-row blocks per workgroup
constexpr int kARows = 16 * kARB;          // weight rows per workgroup
constexpr int kAGroups = 32;               // groups per row, at most (two 16-row A blocks)
constexpr int kAXRow = 272;                // A buffer row: 128 bf16 of a batch + 16-byte pad
constexpr int kAXBytes = kAGroups * kAXRow;
constexpr int kACRow = 144;                // code buffer row: 128 bytes of a pair + 16-byte pad
constexpr int kACBytes = 16 * kACRow;

// One batch pair (256 columns) of a wave's loads: code load i holds rows
// 8 i + l / 8 of the workgroup, bytes 16 (l % 8) of the pair's 128; for batch
// j the lane's two columns 2 l, 2 l + 1 (activations as one bf16 pair, group
// indices).
struct AStage {
  u32x4 cw[2 * kARB];
  uint32_t xv[2];
  int32_t gv[2][2];
};

// Offsets are 32-bit from the arrays' bases (act_mma_ok keeps them below
// 2^31), so that every load takes a uniform base and one lane offset.
struct ARows {
  const uint8_t* cb;              // code words
  const uint8_t* xb;              // activations
  const uint8_t* gb;              // g_idx
  uint32_t c[2 * kARB];           // byte offset of code row 8 i + l / 8 (at most N - 1) + 16 (l % 8)
  uint32_t l4;                    // 4 l: byte offset of the activation pair 2 l, 2 l + 1

  __device__ __forceinline__ ARows(const LinearArgs& a, int64_t n0, int lane) {
    const uint32_t KB = static_cast<uint32_t>(a.K / 2), N1 = static_cast<uint32_t>(a.N - 1);
    cb = a.codes;
    xb = reinterpret_cast<const uint8_t*>(a.x);
    gb = reinterpret_cast<const uint8_t*>(a.g_idx);
#pragma unroll
    for (int i = 0; i < 2 * kARB; ++i)
      c[i] = min(static_cast<uint32_t>(n0) + 8u * i + static_cast<uint32_t>(lane >> 3), N1) * KB + 16u * (lane & 7);
    l4 = 4u * lane;
  }
};

// Pair p of the wave's range p0 .. pl.  A prefetch past the range (the loop
// issues whole rounds) reads, in place of code words, 1 KB of the activations,
// which every wave reads and the cache holds, so that no code line is fetched
// twice; its stage is never computed.
__device__ __forceinline__ void a_issue(const ARows& R, uint32_t p, uint32_t pl, AStage& st) {
  const bool past = p > pl;
  const uint8_t* cbase = past ? R.xb : R.cb;
  p = min(p, pl);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t k0 = 256u * p + 128u * j;   // first column of batch j
    st.xv[j] = *reinterpret_cast<const uint32_t*>(R.xb + (2u * k0 + R.l4));
    const int2 g = *reinterpret_cast<const int2*>(R.gb + (4u * k0 + 2u * R.l4));
    st.gv[j][0] = g.x;
    st.gv[j][1] = g.y;
  }
#pragma unroll
  for (int i = 0; i < 2 * kARB; ++i)   // code words are read once: non-temporal
    st.cw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cbase + (past ? 4u * R.l4 : R.c[i] + 128u * p)));
  __builtin_amdgcn_sched_barrier(0);
}

// Byte offset, within a group row of the A buffer, of batch column c: column
// 8 b + e goes to slot (e % 4) * 2 + e / 4 of its 8-column chunk, the order
// decode_word gives the weights, so the 16 bytes of chunk b are an A operand.
__device__ __forceinline__ uint32_t a_slot(uint32_t c) {
  const uint32_t e = c & 7u;
  return 2u * ((c & ~7u) + ((e & 3u) << 1) + (e >> 2));
}

template <int ZP, int H>
struct AAcc {
  f32x4_t c[kARB][H];   // C[g][n] of block rb, groups 16 h + 4 q + t (lane (n, q), slot t)
  f32x4_t xs[H];        // X_g, the same layout
};

// Batch pair p.  prev[e]: the group whose row holds the lane's column 2 l + e
// of the previous batch (the same position in every batch), cleared before
// the new write.
template <int ZP, int H>
__device__ __forceinline__ void a_compute(const AStage& st, int NG, uint32_t mask, int lane, uint8_t* al, uint8_t* cl,
                                          int (&prev)[2], AAcc<ZP, H>& acc) {
  const int q = lane >> 4, n = lane & 15;
  // code words -> operand layout (lane (n, q) of batch j: row n, chunk 4 j + q)
  uint32_t dw[kARB][2][4];
#pragma unroll
  for (int rb = 0; rb < kARB; ++rb) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<u32x4*>(cl + (8 * h + (lane >> 3)) * kACRow + 16 * (lane & 7)) = st.cw[2 * rb + h];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(cl + n * kACRow + 16 * (4 * j + q));
#pragma unroll
      for (int i = 0; i < 4; ++i) dw[rb][j][i] = v[i];
    }
  }
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    // A for batch j: clear the lane's two previous entries, write the new ones
    const uint32_t s0 = a_slot(2u * lane), s1 = a_slot(2u * lane + 1u);
    *reinterpret_cast<uint16_t*>(al + prev[0] * kAXRow + s0) = 0;
    *reinterpret_cast<uint16_t*>(al + prev[1] * kAXRow + s1) = 0;
    const int g0 = min(max(st.gv[j][0], 0), NG - 1), g1 = min(max(st.gv[j][1], 0), NG - 1);
    *reinterpret_cast<uint16_t*>(al + g0 * kAXRow + s0) = static_cast<uint16_t>(st.xv[j] & 0xFFFFu);
    *reinterpret_cast<uint16_t*>(al + g1 * kAXRow + s1) = static_cast<uint16_t>(st.xv[j] >> 16);
    prev[0] = g0;
    prev[1] = g1;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // step s: lane (m, q) holds columns 32 q + 8 s .. + 7 of group rows 16 h + m
      bf16x8_t av[H];
#pragma unroll
      for (int h = 0; h < H; ++h) av[h] = *reinterpret_cast<const bf16x8_t*>(al + (16 * h + n) * kAXRow + 16 * (4 * q + s));
#pragma unroll
      for (int h = 0; h < H; ++h) acc.xs[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[h], ones, acc.xs[h], 0, 0, 0);
#pragma unroll
      for (int rb = 0; rb < kARB; ++rb) {
        const uint32_t d = ZP == 0 ? dw[rb][j][s] ^ 0x88888888u : dw[rb][j][s];   // signed q -> q + 8
        const bf16x8_t bw = decode_word(d, mask);
#pragma unroll
        for (int h = 0; h < H; ++h) acc.c[rb][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[h], bw, acc.c[rb][h], 0, 0, 0);
      }
    }
  }
}

// The epilogue's scales and zero-points of the lane's row n (of each block)
// and groups 16 h + 4 q + t, loaded with the first pairs so that their latency
// is not exposed at the end.  With NG % 4 == 0 the lane's four groups are one
// 16-byte scale load and one zero-point word (byte zero-points) or half-word
// (packed), kept raw until the epilogue; groups past NG get scale 0.
template <int H, bool V4>
struct AEpi {
  float sc[kARB][H][4];
  uint32_t zw[kARB][H][V4 ? 1 : 4];   // V4 (NG % 4 == 0): the four zero-points' bytes; else each one's byte
};
template <int ZP, int H, bool V4>
__device__ __forceinline__ void a_epilogue_loads(const LinearArgs& a, int64_t n0, int lane, AEpi<H, V4>& ep) {
  const int q = lane >> 4, n = lane & 15;
  const int NG = static_cast<int>(a.NG);
  if constexpr (V4) {
#pragma unroll
    for (int rb = 0; rb < kARB; ++rb) {
      const int64_t row = min(n0 + 16 * rb + n, a.N - 1);
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const int g0 = 16 * h + 4 * q;
        const int gc = min(g0, NG - 4);
        // read once per call: non-temporal
        const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(a.scales + row * a.NG + gc));
#pragma unroll
        for (int t = 0; t < 4; ++t) ep.sc[rb][h][t] = g0 < NG ? v[t] : 0.0f;
        if constexpr (ZP == 1) ep.zw[rb][h][0] = *reinterpret_cast<const uint32_t*>(a.zeros + row * a.NG + gc);
        if constexpr (ZP == 2) ep.zw[rb][h][0] = *reinterpret_cast<const uint16_t*>(a.zeros + row * (a.NG / 2) + gc / 2);
      }
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < kARB; ++rb) {
      const int64_t row = min(n0 + 16 * rb + n, a.N - 1);
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int g = 16 * h + 4 * q + t;
          const int gc = min(g, NG - 1);
          const float sv = a.scales[row * a.NG + gc];
          ep.sc[rb][h][t] = g < NG ? sv : 0.0f;
          ep.zw[rb][h][t] = ZP ? zero_byte<ZP == 2>(a.zeros, row, a.NG, gc) : 8u;
        }
    }
  }
}
// zero-point of slot t of the lane's groups (block rb, half h)
template <int ZP, int H, bool V4>
__device__ __forceinline__ uint32_t a_zero(const AEpi<H, V4>& ep, int rb, int h, int t, uint32_t g) {
  if constexpr (ZP == 0) return 8u;
  if constexpr (V4) {
    if constexpr (ZP == 1) return (ep.zw[rb][h][0] >> (8 * t)) & 0xFFu;
    return (ep.zw[rb][h][0] >> (4 * t)) & 0xFu;   // two per byte: slot t is nibble t of the half-word
  }
  return zero_of<ZP == 2>(ep.zw[rb][h][V4 ? 0 : t], g);
}

// With NG % 4 == 0 the workgroup's 32 rows of scales and zero-points are read
// once as whole lines into LDS tables (wave w: rows 8 w .. 8 w + 7, 16 bytes of
// scales and 4 (2 packed) bytes of zero-points per lane), before the code words,
// so that storing them waits for nothing else; row r of a table at r * 36
// words / bytes puts the 16 rows an epilogue read touches on distinct banks.
constexpr int kASRow = 36;
constexpr int kAZRow = 36;
struct ATabLoad {
  f32x4_t s;
  uint32_t z;
};
template <int ZP>
__device__ __forceinline__ void a_table_issue(const LinearArgs& a, int64_t n0, int w, int lane, ATabLoad& tl) {
  const int NG = static_cast<int>(a.NG);
  const int64_t row = min(n0 + 8 * w + (lane >> 3), a.N - 1);
  const int c = min(lane & 7, NG / 4 - 1);
  tl.s = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(a.scales + row * a.NG + 4 * c));
  if constexpr (ZP == 1) tl.z = *reinterpret_cast<const uint32_t*>(a.zeros + row * a.NG + 4 * c);
  if constexpr (ZP == 2) tl.z = *reinterpret_cast<const uint16_t*>(a.zeros + row * (a.NG / 2) + 2 * c);
}
template <int ZP>
__device__ __forceinline__ void a_table_store(int NG, int w, int lane, const ATabLoad& tl, float* stab, uint8_t* ztab) {
  const int r = 8 * w + (lane >> 3), c = lane & 7;
  if (4 * c < NG) {
    *reinterpret_cast<f32x4_t*>(stab + r * kASRow + 4 * c) = tl.s;
    if constexpr (ZP == 1) *reinterpret_cast<uint32_t*>(ztab + r * kAZRow + 4 * c) = tl.z;
    if constexpr (ZP == 2) *reinterpret_cast<uint16_t*>(ztab + r * kAZRow + 2 * c) = static_cast<uint16_t>(tl.z);
  }
}

template <int ZP, int H, bool V4>
__global__ __launch_bounds__(kAWaves * kWave) void act_mma_kernel(LinearArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t abuf[kAWaves][kAXBytes + kACBytes];
  __shared__ float red[kAWaves - 1][kARB][16];
  __shared__ __attribute__((aligned(16))) float stab[V4 ? kARows * kASRow : 1];
  __shared__ __attribute__((aligned(16))) uint8_t ztab[V4 ? kARows * kAZRow : 1];
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kARows;   // rows past N: computed, not stored
  const int NG = static_cast<int>(a.NG);
  const int nb = static_cast<int>(a.K / 128);
  const int bb = w * nb / kAWaves, be = (w + 1) * nb / kAWaves;   // K % 1024 == 0: whole pairs
  uint8_t* al = abuf[w];
  uint8_t* cl = abuf[w] + kAXBytes;
  const uint32_t mask = nibble_mask();
  const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  AAcc<ZP, H> acc;
  AEpi<H, V4> ep;
#pragma unroll
  for (int h = 0; h < H; ++h) {
    acc.xs[h] = zero4;
#pragma unroll
    for (int rb = 0; rb < kARB; ++rb) acc.c[rb][h] = zero4;
  }

  ATabLoad tl;
  if constexpr (V4) a_table_issue<ZP>(a, n0, w, lane, tl);
  if (bb < be) {
    const ARows R(a, n0, lane);
    const uint32_t p0 = static_cast<uint32_t>(bb) / 2, pl = static_cast<uint32_t>(be - 1) / 2;
    AStage st[4];
    a_issue(R, p0, pl, st[0]);
    a_issue(R, p0 + 1, pl, st[1]);
    a_issue(R, p0 + 2, pl, st[2]);
    if constexpr (V4) a_table_store<ZP>(NG, w, lane, tl, stab, ztab);
    else a_epilogue_loads<ZP, H, V4>(a, n0, lane, ep);
    // the A buffer starts at zero (the wave's own stores precede its reads)
    for (int i = lane; i < kAXBytes / 16; i += kWave) reinterpret_cast<u32x4*>(al)[i] = u32x4{0u, 0u, 0u, 0u};
    int prev[2] = {0, 0};
    // whole rounds of four pairs, with no exit inside the loop body (an exit
    // would leave loads pending on a path back to the loop head, and the wait
    // there would cover every load in flight)
    uint32_t p = p0;
    for (; p + 3 <= pl; p += 4) {
      a_issue(R, p + 3, pl, st[3]);
      a_compute<ZP, H>(st[0], NG, mask, lane, al, cl, prev, acc);
      a_issue(R, p + 4, pl, st[0]);
      a_compute<ZP, H>(st[1], NG, mask, lane, al, cl, prev, acc);
      a_issue(R, p + 5, pl, st[1]);
      a_compute<ZP, H>(st[2], NG, mask, lane, al, cl, prev, acc);
      a_issue(R, p + 6, pl, st[2]);
      a_compute<ZP, H>(st[3], NG, mask, lane, al, cl, prev, acc);
    }
    // the last 0 to 3 pairs are already in st[0 .. 2]
    if (p <= pl) {
      a_compute<ZP, H>(st[0], NG, mask, lane, al, cl, prev, acc);
    }
    if (p + 1 <= pl) {
      a_compute<ZP, H>(st[1], NG, mask, lane, al, cl, prev, acc);
    }
    if (p + 2 <= pl) {
      a_compute<ZP, H>(st[2], NG, mask, lane, al, cl, prev, acc);
    }
  }

  // y partial of row n0 + 16 rb + n: sum over the lane's groups g = 16 h + 4 q + t
  // of s (C - (128 + z) X), then over the lane quarters (fixed order)
  const int q = lane >> 4, n = lane & 15;
  if constexpr (V4) {
    if (bb >= be) a_table_store<ZP>(NG, w, lane, tl, stab, ztab);
    __syncthreads();   // every wave's table rows are written
#pragma unroll
    for (int rb = 0; rb < kARB; ++rb)
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const int r = 16 * rb + n, g0 = 16 * h + 4 * q;
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stab + r * kASRow + g0);
#pragma unroll
        for (int t = 0; t < 4; ++t) ep.sc[rb][h][t] = g0 < NG ? v[t] : 0.0f;
        if constexpr (ZP == 1) ep.zw[rb][h][0] = *reinterpret_cast<const uint32_t*>(ztab + r * kAZRow + g0);
        if constexpr (ZP == 2) ep.zw[rb][h][0] = *reinterpret_cast<const uint16_t*>(ztab + r * kAZRow + g0 / 2);
      }
  } else {
    if (bb >= be) a_epilogue_loads<ZP, H, V4>(a, n0, lane, ep);
  }
  float part[kARB];
#pragma unroll
  for (int rb = 0; rb < kARB; ++rb) {
    float v = 0.0f;
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t g = static_cast<uint32_t>(16 * h + 4 * q + t);
        const float zo = 128.0f + static_cast<float>(a_zero<ZP, H, V4>(ep, rb, h, t, g));
        v = __builtin_fmaf(ep.sc[rb][h][t], acc.c[rb][h][t] - zo * acc.xs[h][t], v);   // sc = 0 for g >= NG
      }
    v += __shfl_xor(v, 16, kWave);
    v += __shfl_xor(v, 32, kWave);
    part[rb] = v;
  }
  if (w > 0 && q == 0) {
#pragma unroll
    for (int rb = 0; rb < kARB; ++rb) red[w - 1][rb][n] = part[rb];
  }
  __syncthreads();
  if (w > 0 || q != 0) return;
#pragma unroll
  for (int rb = 0; rb < kARB; ++rb) {
    const int64_t row = n0 + 16 * rb + n;
    if (row >= a.N) continue;
    float v = part[rb];
#pragma unroll
    for (int ww = 0; ww < kAWaves - 1; ++ww) v += red[ww][rb][n];
    const float bias = a.bias ? bf16_to_f32(a.bias[row]) : 0.0f;
    a.y[row] = static_cast<uint16_t>(f32_to_bf16(v + bias));
  }
}

template <int ZP, bool V4>
hipError_t launch_act_mma3(const LinearArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>((a.N + kARows - 1) / kARows)), block(kAWaves * kWave);
  if (a.NG <= 16) act_mma_kernel<ZP, 1, V4><<<grid, block, 0, s>>>(a);
  else act_mma_kernel<ZP, 2, V4><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}
template <int ZP>
hipError_t launch_act_mma2(const LinearArgs& a, hipStream_t s) {
  return a.NG % 4 == 0 ? launch_act_mma3<ZP, true>(a, s) : launch_act_mma3<ZP, false>(a, s);
}

}  // namespace

// M = 1 with g_idx, at most 32 groups per row, K a multiple of 1024 (every
// wave's quarter of K is whole batch pairs), code offsets below 2^31.
bool act_mma_ok(const LinearArgs& a) {
  return a.M == 1 && a.g_idx != nullptr && a.NG <= kAGroups && a.K % 1024 == 0 &&
         a.N * (a.K / 2) < (int64_t{1} << 31);
}

hipError_t launch_act_mma(const LinearArgs& a, hipStream_t s) {
  if (!a.asym) return launch_act_mma2<0>(a, s);
  return a.zpk ? launch_act_mma2<2>(a, s) : launch_act_mma2<1>(a, s);
}

}  // namespace w4
