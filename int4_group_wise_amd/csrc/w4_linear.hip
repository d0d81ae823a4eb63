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
// The streaming decode GEMV (M = 1, K = 4096) lives in w4_stream.hip, the
// prefill path (M > 16) in w4_gemm.hip.
#include "w4_device.h"
#include "w4_dot.h"
#include "w4_internal.h"
#include "w4_mfma.h"

namespace w4 {
namespace {

constexpr int kGemvWaves = 2;   // waves per workgroup (2, 4, 8, 16 measured: 2 best by ~1.5%)
constexpr int kGemvRows = 4;    // weight rows per wave

// One lane's share of one 2048-column chunk of its wave's rows: the 16 code
// bytes (32 columns) of each row plus that slice's scale and offset
// (128 + zero-point).
struct Slice {
  uint4 cw[kGemvRows];
  float sc[kGemvRows];
  uint32_t zb[kGemvRows];   // raw zero-point byte: converted where it is used, so
                            // that no instruction waits for it right after its load
};

// Row bases are wave-uniform (scalar registers); each load adds one 32-bit
// lane offset, so no per-load 64-bit address registers are needed.
template <bool ASYM>
__device__ __forceinline__ void load_slice(const LinearArgs& a, int64_t row0, int u, Slice& s) {
  const int64_t KB = a.K / 2;
  const uint32_t g = (32u * static_cast<uint32_t>(u)) / static_cast<uint32_t>(a.G);
  const uint32_t coff = 16u * static_cast<uint32_t>(u);
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r) {
    const int64_t n = min(row0 + r, a.N - 1);   // clamped rows are computed, not stored
    const uint8_t* crow = a.codes + n * KB;
    // code words are read once: non-temporal, so they do not displace x
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow + coff));
    s.cw[r] = make_uint4(t[0], t[1], t[2], t[3]);
    s.sc[r] = (a.scales + n * a.NG)[g];
    s.zb[r] = ASYM ? zero_row(a.zeros, n, a.NG, a.zpk)[g] : 8u;
  }
}

// Activations of one lane's 32 columns for MT rows, loaded raw and re-paired
// in place (pair_x order), with their sum per row.
template <int MT>
struct XSlice {
  uint4 q[MT][4];
  float sum[MT];
};

template <int MT>
__device__ __forceinline__ void load_x(const LinearArgs& a, int u, int M, XSlice<MT>& x) {
  const uint32_t off = 64u * static_cast<uint32_t>(u);
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const uint8_t* xrow = reinterpret_cast<const uint8_t*>(a.x + static_cast<int64_t>(min(m, M - 1)) * a.K);
#pragma unroll
    for (int i = 0; i < 4; ++i) x.q[m][i] = *reinterpret_cast<const uint4*>(xrow + off + 16u * i);
  }
}

template <int MT>
__device__ __forceinline__ void pair_xslice(XSlice<MT>& x) {
  const uint32_t ones = 0x3F803F80u;   // bf16 pair (1.0, 1.0)
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t in[4] = {x.q[m][i].x, x.q[m][i].y, x.q[m][i].z, x.q[m][i].w};
      uint32_t xp[4];
      pair_x(in, xp);
#pragma unroll
      for (int p = 0; p < 4; ++p) t = dot2_bf16(xp[p], ones, t);
      x.q[m][i] = make_uint4(xp[0], xp[1], xp[2], xp[3]);
    }
    x.sum[m] = t;
  }
}

template <int MT, bool ASYM>
__device__ __forceinline__ void use_slice(const Slice& s, const XSlice<MT>& x, bool valid, uint32_t mask,
                                          float (&tot)[kGemvRows][MT]) {
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r) {
    const uint32_t flip = ASYM ? 0u : 0x88888888u;
    const uint32_t d[4] = {s.cw[r].x ^ flip, s.cw[r].y ^ flip, s.cw[r].z ^ flip, s.cw[r].w ^ flip};
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t xp[4] = {x.q[m][i].x, x.q[m][i].y, x.q[m][i].z, x.q[m][i].w};
        acc = dot8(d[i], mask, xp, acc);
      }
      const float zo = 128.0f + static_cast<float>(s.zb[r]);
      const float v = s.sc[r] * (acc - zo * x.sum[m]);
      tot[r][m] += valid ? v : 0.0f;
    }
  }
}


// Each round covers two 2048-column chunks.  A lane first issues the loads of
// its activations (L2-resident), then the code words, scales and zero-points
// of both chunks (HBM); loads retire in order, so re-pairing the activations
// waits only for them, and the arithmetic of the first chunk overlaps the
// second chunk's transfer.
template <int MT, bool ASYM>
__global__ __launch_bounds__(kGemvWaves * kWave) void gemv_dot2_kernel(LinearArgs a) {
  const int lane = lane_id();
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kGemvWaves +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = wave * kGemvRows;
  if (row0 >= a.N) return;
  const int units = static_cast<int>(a.K / 32);   // 32-column slices per row
  const int M = static_cast<int>(a.M);
  const uint32_t mask = nibble_mask();

  float tot[kGemvRows][MT];
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) tot[r][m] = 0.0f;

  // lane l ends up with the sum of row row0 + l / 16: its bias is loaded first,
  // so that the epilogue does not wait for a global load.  The load is
  // unconditional (without a bias it reads x[0] and the value is dropped): a
  // branch around it would end the block and wait for the load right there.
  static_assert(kGemvRows == 4, "wave_sum4 reduces four rows");
  const int64_t n_out = row0 + (lane >> 4);
  const uint16_t* bsrc = a.bias ? a.bias + min(n_out, a.N - 1) : a.x;
  const uint32_t braw = *bsrc;   // converted in the epilogue
  __builtin_amdgcn_sched_barrier(0);

  // Slices past the row end (K not a multiple of 4096) load the last slice
  // again and are discarded, so the loads need no branches: a branch would
  // end the basic block and force an early wait for all outstanding loads.
  for (int u0 = 0; u0 < units; u0 += 2 * kWave) {
    const int ua = u0 + lane, ub = u0 + kWave + lane;
    const int ca = min(ua, units - 1), cb = min(ub, units - 1);
    XSlice<MT> xa, xb;
    Slice sa, sb;
    // Issue order = use order (loads retire in order); the scheduling
    // barriers keep the compiler from regrouping them.
    load_x<MT>(a, ca, M, xa);
    load_x<MT>(a, cb, M, xb);
    __builtin_amdgcn_sched_barrier(0);
    load_slice<ASYM>(a, row0, ca, sa);
    __builtin_amdgcn_sched_barrier(0);
    load_slice<ASYM>(a, row0, cb, sb);
    __builtin_amdgcn_sched_barrier(0);
    pair_xslice<MT>(xa);
    use_slice<MT, ASYM>(sa, xa, ua < units, mask, tot);
    pair_xslice<MT>(xb);
    use_slice<MT, ASYM>(sb, xb, ub < units, mask, tot);
  }

#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const float v = wave_sum4(tot[0][m], tot[1][m], tot[2][m], tot[3][m]);
    const float bias = a.bias ? bf16_to_f32(braw) : 0.0f;
    if ((lane & 15) == 0 && n_out < a.N && m < M)
      a.y[static_cast<int64_t>(m) * a.N + n_out] = static_cast<uint16_t>(f32_to_bf16(v + bias));
  }
}

// ---------------------------------------------------------------------------
// Decode GEMV with an act-order g_idx (M <= 4; K = 2048 S P): the columns of
// a group are scattered over the row, so every weight needs its own group's
// scale and zero-point.  The workgroup's rows get a table in LDS holding, for
// every (row, group), the 16 possible bf16 values fp32(v) * s of a nibble (the
// values every other path dequantizes to); a weight is then one LDS read at
// the byte offset of its column's group (from g_idx, computed once per wave
// for all rows) plus its nibble.  Two adjacent columns' values form one bf16
// pair for v_dot2_f32_bf16 against the activations' natural pairs.  Rows,
// slices and the load order are as in the streaming GEMV: a set of P waves
// owns R rows, lane l of wave h takes slices l + 64 (P j + h), every load is
// issued before the table is built.
// ---------------------------------------------------------------------------
constexpr int kActWG = 4;   // waves per workgroup


template <int R, int S, int P, int MT, bool ASYM>
__global__ __launch_bounds__(kActWG * kWave) void gemv_act_kernel(LinearArgs a) {
  static_assert(R >= 1 && R <= 16 && (P == 1 || P == 2), "row set shape");
  constexpr int H = (R + 3) / 4;
  constexpr int SETS = kActWG / P;
  extern __shared__ __attribute__((aligned(16))) uint8_t asm_[];
  __shared__ float red[kActWG][MT][4 * H];
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = w % P, set = w / P;
  const int64_t set0 = static_cast<int64_t>(blockIdx.x) * SETS;   // first row set of the workgroup
  const int64_t row0 = (set0 + set) * R;                          // rows past N: computed, not stored
  const int M = static_cast<int>(a.M);
  const int NG = static_cast<int>(a.NG);
  const int64_t KB = a.K / 2;
  auto slice = [&](int j) -> uint32_t { return static_cast<uint32_t>(lane) + 64u * (P * j + h); };

  // 1. loads: activations, group indices and every row's code words of the lane's slices
  u32x4 xr[MT][S][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < S; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xr[m][j][i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a.x + static_cast<int64_t>(min(m, M - 1)) * a.K) +
                                                      64u * slice(j) + 16 * i);
  u32x4 gq[S][8];
#pragma unroll
  for (int j = 0; j < S; ++j)
#pragma unroll
    for (int q = 0; q < 8; ++q) gq[j][q] = *reinterpret_cast<const u32x4*>(a.g_idx + 32 * slice(j) + 4 * q);
  uint32_t braw[H];
#pragma unroll
  for (int hh = 0; hh < H; ++hh) {
    const int64_t n = min(row0 + 4 * hh + (lane >> 4), a.N - 1);
    braw[hh] = a.bias ? a.bias[n] : a.x[0];
  }
  u32x4 cw[R][S];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t n = min(row0 + r, a.N - 1);
#pragma unroll
    for (int j = 0; j < S; ++j)
      cw[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.codes + n * KB + 16u * slice(j)));
  }

  // 2. the value tables of the workgroup's rows: entry (set, group g, row r,
  //    nibble u) at set NG R 32 + g R 32 + r 32 + 2 u, so that a weight's
  //    address is its column's group offset plus a per-row constant plus 2 u
  constexpr int kGroupBytes = R * 32;
  const int entries = SETS * R * NG;
  for (int e = threadIdx.x; e < entries; e += kActWG * kWave) {
    const int st = e / (R * NG), g = (e / R) % NG, r = e % R;
    const int64_t n = min((set0 + st) * R + r, a.N - 1);
    const float sc = a.scales[n * a.NG + g];
    const int z = ASYM ? static_cast<int>(zero_row(a.zeros, n, a.NG, a.zpk)[g]) : 8;
    uint32_t wv[8];
#pragma unroll
    for (int u = 0; u < 16; u += 2) {
      // value formed in integers (signed codes: (u ^ 8) - 8), one fp32
      // multiply, then bf16 pairs rounded to nearest even (v_cvt_pk_bf16_f32)
      const float v0 = static_cast<float>((ASYM ? u : (u ^ 8)) - z) * sc;
      const float v1 = static_cast<float>((ASYM ? u + 1 : ((u + 1) ^ 8)) - z) * sc;
      wv[u / 2] = __builtin_bit_cast(uint32_t, bf16x2_t{static_cast<__bf16>(v0), static_cast<__bf16>(v1)});
    }
    u32x4* dst = reinterpret_cast<u32x4*>(asm_ + (st * NG + g) * kGroupBytes + 32 * r);
    dst[0] = u32x4{wv[0], wv[1], wv[2], wv[3]};
    dst[1] = u32x4{wv[4], wv[5], wv[6], wv[7]};
  }
  __syncthreads();

  // 3. byte offset of each column's group in this set's table
  const uint32_t set_base = static_cast<uint32_t>(set * NG * kGroupBytes);
  uint32_t goff[S][32];
#pragma unroll
  for (int j = 0; j < S; ++j)
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        goff[j][4 * q + e] = set_base + static_cast<uint32_t>(min(max(static_cast<int>(gq[j][q][e]), 0), NG - 1)) * kGroupBytes;

  // 4. rows: one lookup per weight, a dot2 per column pair and activation row
  float tot[MT][4 * H];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 4 * H; ++r) tot[m][r] = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint8_t* trow = asm_ + 32 * r;
#pragma unroll
    for (int j = 0; j < S; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t d = cw[r][j][i];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t u0 = __builtin_amdgcn_ubfe(d, 8 * p, 4), u1 = __builtin_amdgcn_ubfe(d, 8 * p + 4, 4);
          const uint32_t lo = *reinterpret_cast<const uint16_t*>(trow + goff[j][8 * i + 2 * p] + 2 * u0);
          const uint32_t hi = *reinterpret_cast<const uint16_t*>(trow + goff[j][8 * i + 2 * p + 1] + 2 * u1);
          const uint32_t wp = lo | (hi << 16);
#pragma unroll
          for (int m = 0; m < MT; ++m) tot[m][r] = dot2_bf16(wp, xr[m][j][i][p], tot[m][r]);
        }
      }
  }

  // 5. wave sums (lane l: row row0 + 4 hh + l / 16), the two waves of a set
  //    added in a fixed order, bias, store
  float v[MT][H];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int hh = 0; hh < H; ++hh)
      v[m][hh] = wave_sum4(tot[m][4 * hh], tot[m][4 * hh + 1], tot[m][4 * hh + 2], tot[m][4 * hh + 3]);
  if constexpr (P == 2) {
    if (h == 1 && (lane & 15) == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int hh = 0; hh < H; ++hh) red[w][m][4 * hh + (lane >> 4)] = v[m][hh];
    }
    __syncthreads();
    if (h == 1) return;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int hh = 0; hh < H; ++hh) v[m][hh] += red[w + 1][m][4 * hh + (lane >> 4)];
  }
#pragma unroll
  for (int hh = 0; hh < H; ++hh) {
    const int64_t n = row0 + 4 * hh + (lane >> 4);
    const float bias = a.bias ? bf16_to_f32(braw[hh]) : 0.0f;
    if ((lane & 15) == 0 && 4 * hh + (lane >> 4) < R && n < a.N) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < M) a.y[static_cast<int64_t>(m) * a.N + n] = static_cast<uint16_t>(f32_to_bf16(v[m][hh] + bias));
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core decode kernel (M <= 4): v_mfma_f32_16x16x32_bf16 with the
// activations as the 16-row A operand (rows m >= M are padding) and 16 weight
// rows as the B operand.  The only per-weight VALU work is the nibble -> bf16
// decode (7 instructions per 8 weights); the multiply-adds run on the matrix
// cores.
//
// Operand layout: lane l serves weight row n = l % 16 and column quarter
// q = l / 16.  Per 128-column block it holds 16 code bytes (32 columns) of its
// row; dword i feeds MFMA i.  Without transposition MFMA i sums columns
// {kb + 32q + 8i + e}, spanning the whole block (fine for G >= 128).  For
// G = 32 or 64 the four dwords are transposed across the lane quarters
// (v_permlane32_swap + v_permlane16_swap), after which MFMA i sums the 32
// contiguous columns kb + 32i .. kb + 32i + 31, a single group.
//
// Memory access: in that layout the four lanes of a row are 16 apart, so a
// load would touch a different cache line in every lane.  Instead lanes
// 4r..4r+3 load the 64 contiguous bytes of row r (16 rows per instruction,
// one line per lane quad), and each block is re-laid out through a 1 KB
// wave-private LDS scratch.  Scales and zero-points of the wave's 16 rows are
// loaded the same way (consecutive lanes, consecutive groups) into an LDS
// table.
//
// Workgroup = 4 waves on one 16-row tile, each wave a quarter of K; the
// partial tiles are summed in LDS at the end.  The activations (re-paired to
// the decode's slot order, plus their sums per 32 columns) are staged once in
// LDS.  Load order is activations, scale/zero tables, code words: loads retire
// in order, so the staging waits only for the first two, and the barrier
// before the arithmetic does not wait for outstanding global loads.
// ---------------------------------------------------------------------------

constexpr int kTileWaves = 4;
constexpr int kMfmaKR = 8;           // k-blocks (128 columns) per round

// Groups one wave's round can touch in a row: KR blocks of 128 columns hold
// KR * 128 / G groups for G <= 128, at most KR + 1 for G > 128.
constexpr int kMaxTileGroups = 4 * kMfmaKR;

// LDS layout (bytes) for a K of `kc` columns and MT activation rows:
//   x      paired activation chunks, row m at m * xrow, chunk c at + 16 c,
//          xrow = 2 kc + 16 (the pad spreads rows over the banks);
//   xs     float sums per row and 32-column unit, [MT][kc / 32];
//   xsb    float sums per row and 128-column block, [MT][kc / 128];
//   wave   per wave: 1 KB code scratch, scale table [16][kMaxTileGroups]
//          floats, zero table [16][kMaxTileGroups] bytes;
//   red    cross-wave reduction [kTileWaves][MT][16] floats.
struct XLayout {
  uint32_t xrow, xs_off, xsb_off, wave_off, wave_bytes, red_off, bytes;
};

__host__ __device__ inline XLayout x_layout(int MT, int64_t kc) {
  XLayout L;
  L.xrow = static_cast<uint32_t>(2 * kc + 16);
  L.xs_off = MT * L.xrow;
  L.xsb_off = L.xs_off + static_cast<uint32_t>(MT * (kc / 32) * 4);
  L.wave_off = (L.xsb_off + static_cast<uint32_t>(MT * (kc / 128) * 4) + 15u) & ~15u;
  L.wave_bytes = 1024 + 16 * kMaxTileGroups * 4 + 16 * kMaxTileGroups;
  L.red_off = L.wave_off + kTileWaves * L.wave_bytes;
  L.bytes = L.red_off + kTileWaves * MT * 16 * 4;
  return L;
}

template <int MT, bool ASYM, bool TR, int GU>
__global__ __launch_bounds__(kTileWaves * kWave, 4) void skinny_mfma_kernel(LinearArgs a, int kpw) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int KR = kMfmaKR;
  const int K = static_cast<int>(a.K);
  const int M = static_cast<int>(a.M);
  const XLayout L = x_layout(MT, K);
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, q = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;   // rows past N are clamped: computed, not stored
  const int nkb = K / 128;
  const int kb0 = min(nkb, w * kpw), kb1 = min(nkb, kb0 + kpw);
  const int64_t KB = a.K / 2;
  const uint32_t G = static_cast<uint32_t>(a.G);
  uint8_t* wave_lds = smem + L.wave_off + w * L.wave_bytes;
  u32x4* scratch = reinterpret_cast<u32x4*>(wave_lds);
  float* stab = reinterpret_cast<float*>(wave_lds + 1024);
  uint8_t* ztab = wave_lds + 1024 + 16 * kMaxTileGroups * 4;

  // 1. activations: 32-column units (64 bytes of one row), MT per thread per
  //    batch.  All batches but the last are staged at once; the last one is
  //    loaded, then the other loads are issued, then it is staged.
  const int units = K / 32;
  const int xu_total = MT * units;
  const int nbatch = (xu_total + 256 * MT - 1) / (256 * MT);
  u32x4 xr[MT][4];
  auto load_x_batch = [&](int bt) {
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int t = min(bt * 256 * MT + static_cast<int>(threadIdx.x) + 256 * j, xu_total - 1);
      const int m = t / units, u = t % units;
      const uint8_t* src = reinterpret_cast<const uint8_t*>(a.x + static_cast<int64_t>(min(m, M - 1)) * a.K) + 64u * u;
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[j][i] = *reinterpret_cast<const u32x4*>(src + 16 * i);
    }
  };
  auto stage_x_batch = [&](int bt) {
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int t = bt * 256 * MT + static_cast<int>(threadIdx.x) + 256 * j;
      if (t < xu_total) {
        const int m = t / units, u = t % units;
        const bool live = m < M;
        const uint32_t ones = 0x3F803F80u;
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t in[4] = {xr[j][i][0], xr[j][i][1], xr[j][i][2], xr[j][i][3]};
          uint32_t xp[4];
          pair_x(in, xp);
#pragma unroll
          for (int p = 0; p < 4; ++p) sum = dot2_bf16(xp[p], ones, sum);
          const u32x4 pv = {xp[0], xp[1], xp[2], xp[3]};
          *reinterpret_cast<u32x4*>(smem + m * L.xrow + 64u * u + 16 * i) = live ? pv : u32x4{0u, 0u, 0u, 0u};
        }
        reinterpret_cast<float*>(smem + L.xs_off)[t] = live ? sum : 0.0f;
      }
    }
  };
  for (int bt = 0; bt + 1 < nbatch; ++bt) {
    load_x_batch(bt);
    stage_x_batch(bt);
  }
  load_x_batch(nbatch - 1);

  // 2. per round: the scale/zero table of the wave's 16 rows (consecutive
  //    lanes read consecutive groups of a row), then the code words: load j
  //    brings k-block j, lane quad r holding the 64 bytes of row r.
  const uint32_t rq = static_cast<uint32_t>(lane >> 2), cq = static_cast<uint32_t>(lane & 3);
  const uint32_t rload = static_cast<uint32_t>(min(static_cast<int64_t>(rq), a.N - 1 - n0));
  const uint8_t* cbase = a.codes + n0 * KB;
  const float* sbase = a.scales + n0 * a.NG;
  u32x4 cw[KR];
  // table loads: lane quad r covers row r, lane cq takes groups cq, cq + 4, ...
  constexpr int kTG = GU == 1 ? KR + 1 : KR * GU;     // groups per row per round, at most
  constexpr int kTabLoads = (kTG + 3) / 4;
  float tabs[kTabLoads];
  uint32_t tabz[kTabLoads];
  int g_first = 0, ngt = 1;
  auto issue = [&](int kbs) {
    const int kbl = min(kbs + KR, kb1) - 1;          // last k-block of the round
    g_first = static_cast<int>((128u * kbs) / G);
    ngt = static_cast<int>((128u * kbl + 127u) / G) - g_first + 1;
    const uint32_t trow = rload * static_cast<uint32_t>(a.NG) + static_cast<uint32_t>(g_first);
#pragma unroll
    for (int j = 0; j < kTabLoads; ++j) {
      const uint32_t gg = static_cast<uint32_t>(min(4 * j + static_cast<int>(cq), ngt - 1));
      tabs[j] = sbase[trow + gg];
      tabz[j] = ASYM ? zero_row(a.zeros, n0 + rload, a.NG, a.zpk)[g_first + gg] : 8u;
    }
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      const uint32_t kb = static_cast<uint32_t>(min(kbs + j, nkb - 1));
      cw[j] = __builtin_nontemporal_load(   // code words are read once
          reinterpret_cast<const u32x4*>(cbase + rload * static_cast<uint32_t>(KB) + 64u * kb + 16u * cq));
    }
  };
  auto store_tab = [&]() {
#pragma unroll
    for (int j = 0; j < kTabLoads; ++j) {
      const int gg = 4 * j + static_cast<int>(cq);
      if (gg < ngt) {
        stab[rq * kMaxTileGroups + gg] = tabs[j];
        ztab[rq * kMaxTileGroups + gg] = static_cast<uint8_t>(tabz[j]);
      }
    }
  };
  issue(kb0);
  __builtin_amdgcn_sched_barrier(0);

  // 3. stage the last activation batch and the first table, sums per block
  stage_x_batch(nbatch - 1);
  store_tab();
  __syncthreads();
  for (int t = threadIdx.x; t < MT * (K / 128); t += kTileWaves * kWave) {
    const float* xs4 = reinterpret_cast<const float*>(smem + L.xs_off) + 4 * t;
    reinterpret_cast<float*>(smem + L.xsb_off)[t] = (xs4[0] + xs4[1]) + (xs4[2] + xs4[3]);
  }
  __syncthreads();

  // 4. arithmetic.  A-operand row of this lane: output rows are independent,
  //    so lanes whose activation row is absent (m >= MT) may read any staged
  //    row; their output rows are discarded.
  const uint32_t a_base = (n < MT ? n : 0) * L.xrow;
  const uint32_t mask = nibble_mask();
  const float* xs = reinterpret_cast<const float*>(smem + L.xs_off);
  const float* xsb = reinterpret_cast<const float*>(smem + L.xsb_off);
  float out[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) out[t] = 0.0f;
  const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int kbs = kb0; kbs < kb1; kbs += KR) {
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      const int kb = kbs + j;
      if (kb < kb1) {
        // re-lay the block out: row-major in, operand layout out
        scratch[rq * 4 + cq] = cw[j];
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): the wave's own LDS writes
        const u32x4 v = scratch[n * 4 + q];
        uint32_t d[4] = {v[0], v[1], v[2], v[3]};
        if constexpr (!ASYM) {
#pragma unroll
          for (int i = 0; i < 4; ++i) d[i] ^= 0x88888888u;
        }
        if constexpr (TR) transpose_quarters(d);
        f32x4_t acc[GU];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t chunk = TR ? (16u * kb + 4u * i + q) : (16u * kb + 4u * q + i);
          const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(smem + a_base + 16u * chunk);
          const int gi = i / (4 / GU);
          acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, decode_word(d[i], mask),
                                                            (i % (4 / GU)) == 0 ? zero4 : acc[gi], 0, 0, 0);
        }
        // group correction: out += s * (acc - (128 + z) * sum_x); output rows
        // 4 (l / 16) + t, so for M <= 4 only the first quarter's t < M matter
#pragma unroll
        for (int gi = 0; gi < GU; ++gi) {
          const int col = 128 * kb + (128 / GU) * gi;
          const int gg = col / static_cast<int>(G) - g_first;
          const float sc = stab[n * kMaxTileGroups + gg];
          const float zo = 128.0f + static_cast<float>(ztab[n * kMaxTileGroups + gg]);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const float sx = GU == 1 ? xsb[t * (K / 128) + kb] : 0.0f;
            float sxu = 0.0f;
            if constexpr (GU > 1) {
#pragma unroll
              for (int uu = 0; uu < 4 / GU; ++uu) sxu += xs[t * units + 4 * kb + gi * (4 / GU) + uu];
            }
            out[t] += sc * (acc[gi][t] - zo * (GU == 1 ? sx : sxu));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // bound register use: one k-block in flight
    }
    if (kbs + KR < kb1) {
      issue(kbs + KR);
      store_tab();
    }
  }

  // 5. sum the four K quarters and store
  float* red = reinterpret_cast<float*>(smem + L.red_off);
  if (lane < 16) {
#pragma unroll
    for (int t = 0; t < MT; ++t) red[(w * MT + t) * 16 + n] = out[t];
  }
  __syncthreads();
  if (w == 0 && lane < 16 && n0 + n < a.N) {
    const float b = a.bias ? bf16_to_f32(a.bias[n0 + n]) : 0.0f;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < M) {
        float v = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kTileWaves; ++ww) v += red[(ww * MT + t) * 16 + n];
        a.y[static_cast<int64_t>(t) * a.N + n0 + n] = static_cast<uint16_t>(f32_to_bf16(v + b));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core batched-decode kernel (4 < M <= 16).  The same operand scheme
// as skinny_mfma_kernel (activations = 16-row A operand, 16 weight rows = B
// operand, nibbles decoded to 128 + u, per-group correction), organised for
// activation reuse: a workgroup's 4 waves own 4 different 16-row tiles and
// walk K together in batches of kRowsKB blocks of 128 columns; each batch's
// activations [16 rows x 512 columns] are staged once in LDS (re-paired, with
// sums per 32 columns) and read by all 4 waves.  Batches are double-buffered:
// batch b + 1 is loaded (activations, scale/zero tables, code words, in that
// order) while batch b is computed.  Code words are loaded straight into the
// operand layout (lane l: row l % 16, 16-byte quarter l / 16 of a block).
// ---------------------------------------------------------------------------
constexpr int kRowsWaves = 4;
constexpr int kRowsKB = 4;                      // 128-column blocks per batch
constexpr int kRowsTG = 16;                     // table groups per row per batch, at most
constexpr int kRowsTS = kRowsTG + 1;            // table row stride (odd: rows on distinct banks)
// staged activations: chunk c (16 bytes) of a batch row is stored at chunk
// x_swz(c) = c with its low two bits rotated by bits 3..4, so the 16 lanes
// that stage one row (64-byte units) write distinct banks
__host__ __device__ constexpr uint32_t x_swz(uint32_t c) {
  return (c & ~3u) | (((c & 3u) + ((c >> 3) & 3u)) & 3u);
}
// activation sums: row m, unit u at m * (kRowsKB * 4) + (u ^ xs_swz(m)); the XOR keeps
// aligned groups of 4 together and puts the 4 lane quarters' rows on distinct banks
__device__ __forceinline__ int xs_swz(int m) { return 4 * ((m >> 2) & 3); }

struct RowsLayout {
  uint32_t xrow, xbuf, xs_off, xsbuf, wave_off, wave_bytes, bytes;
};

__host__ __device__ inline RowsLayout rows_layout() {
  RowsLayout L;
  L.xrow = kRowsKB * 128 * 2 + 16;              // one activation row of a batch (+ bank pad)
  L.xbuf = 16 * L.xrow;
  L.xs_off = 2 * L.xbuf;
  L.xsbuf = 16 * kRowsKB * 4 * 4;               // [16 rows][kRowsKB * 4 units] floats
  L.wave_off = L.xs_off + 2 * L.xsbuf;
  L.wave_bytes = (16 * kRowsTS * 4 + 16 * kRowsTS + 15) & ~15;
  L.bytes = L.wave_off + kRowsWaves * L.wave_bytes;
  return L;
}

struct RowsRegs {
  u32x4 x[4];          // this thread's staged activation unit (64 bytes)
  u32x4 cw[kRowsKB];   // code words, load j = block j of the batch
  float ts[4];         // scale table entries
  uint32_t tz[4];      // zero-point table entries
};

template <bool ASYM>
__device__ __forceinline__ void rows_issue(const LinearArgs& a, int b, int nkb, int64_t n0,
                                           int lane, RowsRegs& R) {
  const int M = static_cast<int>(a.M);
  const int K = static_cast<int>(a.K);
  const uint32_t G = static_cast<uint32_t>(a.G);
  // activations: thread t stages row t / 16, unit t % 16 of the batch
  const int t = threadIdx.x;
  const int xm = min(t >> 4, M - 1);
  const int col = min(b * kRowsKB * 128 + 32 * (t & 15), K - 32);
  const uint8_t* xs = reinterpret_cast<const uint8_t*>(a.x + static_cast<int64_t>(xm) * a.K + col);
#pragma unroll
  for (int i = 0; i < 4; ++i) R.x[i] = *reinterpret_cast<const u32x4*>(xs + 16 * i);
  __builtin_amdgcn_sched_barrier(0);
  // scale / zero-point table: lane quad r = row r, lane cq takes groups cq + 4 i
  const uint32_t rq = static_cast<uint32_t>(lane >> 2), cq = static_cast<uint32_t>(lane & 3);
  const uint32_t rload = static_cast<uint32_t>(min(static_cast<int64_t>(rq), a.N - 1 - n0));
  const int kbf = b * kRowsKB, kbl = min(kbf + kRowsKB, nkb) - 1;
  const int g_first = static_cast<int>((128u * kbf) / G);
  const int ngt = static_cast<int>((128u * kbl + 127u) / G) - g_first + 1;
  const uint32_t trow = (static_cast<uint32_t>(n0) + rload) * static_cast<uint32_t>(a.NG) + static_cast<uint32_t>(g_first);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t gg = static_cast<uint32_t>(min(4 * i + static_cast<int>(cq), ngt - 1));
    R.ts[i] = a.scales[trow + gg];
    R.tz[i] = ASYM ? zero_row(a.zeros, n0 + rload, a.NG, a.zpk)[g_first + gg] : 8u;
  }
  __builtin_amdgcn_sched_barrier(0);
  // code words, straight into the operand layout: lane l holds row l % 16,
  // 16-byte quarter l / 16 of each 128-column block (the 16 rows' 64 bytes
  // per instruction; an LDS relayout of row-contiguous loads measured 2%
  // slower)
  const uint32_t rd = static_cast<uint32_t>(min(static_cast<int64_t>(lane & 15), a.N - 1 - n0));
  const uint8_t* crow = a.codes + (n0 + rd) * (a.K / 2);
#pragma unroll
  for (int j = 0; j < kRowsKB; ++j) {
    const uint32_t kb = static_cast<uint32_t>(min(kbf + j, nkb - 1));
    R.cw[j] = __builtin_nontemporal_load(   // code words are read once
        reinterpret_cast<const u32x4*>(crow + 64u * kb + 16u * static_cast<uint32_t>(lane >> 4)));
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Stage batch b's activations into buffer b % 2 and this wave's tables.
__device__ __forceinline__ void rows_stage(const LinearArgs& a, int b, int lane, const RowsRegs& R,
                                           uint8_t* smem, const RowsLayout& L, uint8_t* wave_lds) {
  const int M = static_cast<int>(a.M);
  const int K = static_cast<int>(a.K);
  const int t = threadIdx.x;
  const int m = t >> 4, uu = t & 15;
  const bool live = m < M && b * kRowsKB * 128 + 32 * uu < K;
  const uint32_t ones = 0x3F803F80u;
  uint8_t* xb = smem + (b & 1) * L.xbuf + m * L.xrow + 64 * uu;
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t in[4] = {R.x[i][0], R.x[i][1], R.x[i][2], R.x[i][3]};
    uint32_t xp[4];
    pair_x(in, xp);
#pragma unroll
    for (int p = 0; p < 4; ++p) sum = dot2_bf16(xp[p], ones, sum);
    *reinterpret_cast<u32x4*>(xb - 64 * uu + 16 * x_swz(4 * uu + i)) =
        live ? u32x4{xp[0], xp[1], xp[2], xp[3]} : u32x4{0u, 0u, 0u, 0u};
  }
  reinterpret_cast<float*>(smem + L.xs_off + (b & 1) * L.xsbuf)[m * (kRowsKB * 4) + (uu ^ xs_swz(m))] = live ? sum : 0.0f;
  const int rq = lane >> 2, cq = lane & 3;
  float* stab = reinterpret_cast<float*>(wave_lds);
  uint8_t* ztab = wave_lds + 16 * kRowsTS * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    stab[rq * kRowsTS + 4 * i + cq] = R.ts[i];
    ztab[rq * kRowsTS + 4 * i + cq] = static_cast<uint8_t>(R.tz[i]);
  }
}

template <bool ASYM, bool TR, int GU>
__device__ __forceinline__ void rows_compute(const LinearArgs& a, int b, int nkb, int lane, uint32_t mask,
                                             const RowsRegs& R, const uint8_t* smem, const RowsLayout& L,
                                             uint8_t* wave_lds, float (&out)[4]) {
  const uint32_t G = static_cast<uint32_t>(a.G);
  const int n = lane & 15, q = lane >> 4;
  const float* stab = reinterpret_cast<const float*>(wave_lds);
  const uint8_t* ztab = wave_lds + 16 * kRowsTS * 4;
  const uint8_t* xa = smem + (b & 1) * L.xbuf + n * L.xrow;          // A row n (zero rows for m >= M)
  const float* xs = reinterpret_cast<const float*>(smem + L.xs_off + (b & 1) * L.xsbuf);
  const int kbf = b * kRowsKB;
  const int g_first = static_cast<int>((128u * kbf) / G);
  const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < kRowsKB; ++j) {
    if (kbf + j < nkb) {
      const u32x4 v = R.cw[j];   // row n, columns 32 q .. 32 q + 31 of the block
      uint32_t d[4] = {v[0], v[1], v[2], v[3]};
      if constexpr (!ASYM) {
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] ^= 0x88888888u;
      }
      if constexpr (TR) transpose_quarters(d);
      f32x4_t acc[GU];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t chunk = TR ? (16u * j + 4u * i + q) : (16u * j + 4u * q + i);
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(xa + 16u * x_swz(chunk));
        const int gi = i / (4 / GU);
        acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, decode_word(d[i], mask),
                                                          (i % (4 / GU)) == 0 ? zero4 : acc[gi], 0, 0, 0);
      }
#pragma unroll
      for (int gi = 0; gi < GU; ++gi) {
        // table index of the group: G = 128 / GU for GU > 1, so the batch's
        // groups start at g_first = GU kbf and this one is GU j + gi
        int gg;
        if constexpr (GU > 1) {
          gg = GU * j + gi;
        } else {
          gg = (128 * (kbf + j)) / static_cast<int>(G) - g_first;
        }
        const float sc = stab[n * kRowsTS + gg];
        // 128 + zero-point (signed codes: 128 + 8)
        const float zo = ASYM ? 128.0f + static_cast<float>(ztab[n * kRowsTS + gg]) : 136.0f;
        const int u0 = 4 * j + gi * (4 / GU);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int m = 4 * q + t;                    // output row of acc[gi][t]
          float sx = xs[m * (kRowsKB * 4) + (u0 ^ xs_swz(m))];
#pragma unroll
          for (int uu = 1; uu < 4 / GU; ++uu) sx += xs[m * (kRowsKB * 4) + ((u0 + uu) ^ xs_swz(m))];
          out[t] += sc * (acc[gi][t] - zo * sx);
        }
      }
    }
  }
}

// Split-K: blockIdx.y = split s of `splits` takes batches [s nbat / splits,
// (s + 1) nbat / splits); with more than one split the fp32 partial tiles go to
// a.partial [splits][M][N] and rows_reduce_kernel adds them in split order.
template <bool ASYM, bool TR, int GU>
__global__ __launch_bounds__(kRowsWaves * kWave, 2) void skinny_rows_kernel(LinearArgs a, int splits) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const RowsLayout L = rows_layout();
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * (16 * kRowsWaves) + 16 * w;  // rows past N are clamped
  const int64_t n0c = min(n0, a.N - 1);
  uint8_t* wave_lds = smem + L.wave_off + w * L.wave_bytes;
  const int nkb = static_cast<int>(a.K / 128);
  const int nbat = (nkb + kRowsKB - 1) / kRowsKB;
  const uint32_t mask = nibble_mask();
  float out[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  const int bb = static_cast<int>(static_cast<int64_t>(blockIdx.y) * nbat / splits);
  const int be = static_cast<int>(static_cast<int64_t>(blockIdx.y + 1) * nbat / splits);
  RowsRegs ra, rb;
  rows_issue<ASYM>(a, bb, nkb, n0c, lane, ra);
  rows_stage(a, bb, lane, ra, smem, L, wave_lds);
  __syncthreads();
  for (int b = bb; b < be; b += 2) {
    if (b + 1 < be) rows_issue<ASYM>(a, b + 1, nkb, n0c, lane, rb);
    rows_compute<ASYM, TR, GU>(a, b, nkb, lane, mask, ra, smem, L, wave_lds, out);
    if (b + 1 >= be) break;
    rows_stage(a, b + 1, lane, rb, smem, L, wave_lds);
    __syncthreads();
    if (b + 2 < be) rows_issue<ASYM>(a, b + 2, nkb, n0c, lane, ra);
    rows_compute<ASYM, TR, GU>(a, b + 1, nkb, lane, mask, rb, smem, L, wave_lds, out);
    if (b + 2 >= be) break;
    rows_stage(a, b + 2, lane, ra, smem, L, wave_lds);
    __syncthreads();
  }

  // lane holds output rows m = 4 q + t of weight row n0 + n
  const int n = lane & 15, q = lane >> 4;
  if (splits > 1) {
    if (n0 + n < a.N) {
      float* part = a.partial + static_cast<int64_t>(blockIdx.y) * a.M * a.N;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = 4 * q + t;
        if (m < a.M) part[static_cast<int64_t>(m) * a.N + n0 + n] = out[t];
      }
    }
    return;
  }
  if (n0 + n < a.N) {
    const float bias = a.bias ? bf16_to_f32(a.bias[n0 + n]) : 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int m = 4 * q + t;
      if (m < a.M) a.y[static_cast<int64_t>(m) * a.N + n0 + n] = static_cast<uint16_t>(f32_to_bf16(out[t] + bias));
    }
  }
}

// y[m, n] = bf16(sum over splits s = 0 .. S-1 of partial[s][m][n] + b[n]),
// one thread per output, the splits added in order.
__global__ __launch_bounds__(256) void rows_reduce_kernel(const float* __restrict__ partial, int splits, int64_t M,
                                                          int64_t N, const uint16_t* __restrict__ bias,
                                                          uint16_t* __restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= M * N) return;
  float t = 0.0f;
  for (int sp = 0; sp < splits; ++sp) t += partial[static_cast<int64_t>(sp) * M * N + i];
  const float b = bias ? bf16_to_f32(bias[i % N]) : 0.0f;
  y[i] = static_cast<uint16_t>(f32_to_bf16(t + b));
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
  const ZeroRow zrow = zero_row(ASYM ? a.zeros : nullptr, n, a.NG, a.zpk);
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

// Act-order decode: rows per set as the streaming GEMV; P = 2 waves per set
// when K is a multiple of 4096 (S = K / 4096 slices per wave), else P = 1
// with K = 2048 (one slice).
template <int R, int S, int P, int MT>
hipError_t launch_act4(const LinearArgs& a, hipStream_t s) {
  constexpr int sets_per_wg = kActWG / P;
  const int64_t sets = (a.N + R - 1) / R;
  const size_t lds = static_cast<size_t>(sets_per_wg) * R * 32 * a.NG;
  const dim3 grid(static_cast<uint32_t>((sets + sets_per_wg - 1) / sets_per_wg)), block(kActWG * kWave);
  if (a.asym) gemv_act_kernel<R, S, P, MT, true><<<grid, block, lds, s>>>(a);
  else gemv_act_kernel<R, S, P, MT, false><<<grid, block, lds, s>>>(a);
  return hipGetLastError();
}

template <int S, int P, int MT>
hipError_t launch_act3(const LinearArgs& a, hipStream_t s) {
  switch (stream_rows(a.N)) {
    case 2: return launch_act4<2, S, P, MT>(a, s);
    case 4: return launch_act4<4, S, P, MT>(a, s);
    case 7: return launch_act4<7, S, P, MT>(a, s);
    default: return launch_act4<8, S, P, MT>(a, s);
  }
}

template <int MT>
hipError_t launch_act2(const LinearArgs& a, hipStream_t s) {
  if (a.K == 2048) return launch_act3<1, 1, MT>(a, s);
  if (a.K == 4096) return launch_act3<1, 2, MT>(a, s);
  return launch_act3<2, 2, MT>(a, s);   // K = 8192
}

// Act-order decode kernel: g_idx, M <= 4, K of 2048, 4096 or 8192, and a
// value table of at most 128 groups per row (LDS: 4 sets x 8 rows x 4 KB).
bool act_ok(const LinearArgs& a) {
  return a.g_idx != nullptr && a.M <= 4 && (a.K == 2048 || a.K == 4096 || a.K == 8192) && a.NG <= 128;
}

hipError_t launch_act(const LinearArgs& a, hipStream_t s) {
  if (a.M == 1) return launch_act2<1>(a, s);
  if (a.M == 2) return launch_act2<2>(a, s);
  return launch_act2<4>(a, s);
}

template <int MT, bool ASYM, bool TR, int GU>
hipError_t launch_mfma4(const LinearArgs& a, hipStream_t s) {
  const int nkb = static_cast<int>(a.K / 128);
  const int kpw = (nkb + kTileWaves - 1) / kTileWaves;
  const XLayout L = x_layout(MT, a.K);
  const dim3 grid(static_cast<uint32_t>((a.N + 15) / 16)), block(kTileWaves * kWave);
  skinny_mfma_kernel<MT, ASYM, TR, GU><<<grid, block, L.bytes, s>>>(a, kpw);
  return hipGetLastError();
}

template <int MT, bool ASYM>
hipError_t launch_mfma3(const LinearArgs& a, hipStream_t s) {
  if (a.G == 32) return launch_mfma4<MT, ASYM, true, 4>(a, s);
  if (a.G == 64) return launch_mfma4<MT, ASYM, true, 2>(a, s);
  return launch_mfma4<MT, ASYM, false, 1>(a, s);
}

template <int MT>
hipError_t launch_mfma2(const LinearArgs& a, hipStream_t s) {
  return a.asym ? launch_mfma3<MT, true>(a, s) : launch_mfma3<MT, false>(a, s);
}

// The matrix-core decode kernel covers contiguous groups of 32, 64 or a
// multiple of 128 columns, K a multiple of 128, M <= 4, and activations that
// fit the 64 KB LDS staging area.
bool mfma_ok(const LinearArgs& a) {
  if (a.g_idx != nullptr || a.K % 128 != 0 || a.M > 4) return false;
  if (!(a.G == 32 || a.G == 64 || a.G % 128 == 0)) return false;
  const int MT = a.M == 1 ? 1 : a.M == 2 ? 2 : 4;
  return x_layout(MT, a.K).bytes <= 65536;
}

// Split-K count for the batched decode kernel: doubled (within the number of
// batches) until the grid holds at least kRowsMinWaves waves, four per SIMD.
constexpr int64_t kRowsMinWaves = 4096;
int rows_splits(int64_t N, int64_t K) {
  const int64_t waves = (N + 15) / 16;
  const int64_t nbat = (K / 128 + kRowsKB - 1) / kRowsKB;
  int sp = 1;
  while (waves * sp < kRowsMinWaves && 2 * sp <= nbat) sp *= 2;
  return sp;
}

template <bool ASYM, bool TR, int GU>
hipError_t launch_rows3(const LinearArgs& a, hipStream_t s) {
  const RowsLayout L = rows_layout();
  const int splits = a.partial ? rows_splits(a.N, a.K) : 1;
  const dim3 grid(static_cast<uint32_t>((a.N + 16 * kRowsWaves - 1) / (16 * kRowsWaves)), static_cast<uint32_t>(splits));
  skinny_rows_kernel<ASYM, TR, GU><<<grid, dim3(kRowsWaves * kWave), L.bytes, s>>>(a, splits);
  if (splits > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    rows_reduce_kernel<<<dim3(static_cast<uint32_t>((a.M * a.N + 255) / 256)), dim3(256), 0, s>>>(
        a.partial, splits, a.M, a.N, a.bias, a.y);
  }
  return hipGetLastError();
}

template <bool ASYM>
hipError_t launch_rows2(const LinearArgs& a, hipStream_t s) {
  if (a.G == 32) return launch_rows3<ASYM, true, 4>(a, s);
  if (a.G == 64) return launch_rows3<ASYM, true, 2>(a, s);
  return launch_rows3<ASYM, false, 1>(a, s);
}

// Batched decode on the matrix cores: contiguous groups of 32, 64 or a
// multiple of 128 columns, K a multiple of 128, 4 < M <= 16.
bool rows_shape_ok(int64_t M, int64_t K, int64_t G, bool has_g_idx) {
  return !has_g_idx && K % 128 == 0 && M > 4 && M <= 16 && (G == 32 || G == 64 || G % 128 == 0);
}
bool rows_ok(const LinearArgs& a) { return rows_shape_ok(a.M, a.K, a.G, a.g_idx != nullptr); }

bool dot2_ok(const LinearArgs& a) {
  return a.g_idx == nullptr && a.G % 32 == 0 && a.K % 32 == 0 && a.M <= 4;
}

}  // namespace

bool skinny_supported(const LinearArgs& a) { return a.M >= 1 && a.M <= 16; }

size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G, bool has_g_idx, bool asym) {
  if (batched_shape_ok(N, M, K, G, has_g_idx, asym) || !rows_shape_ok(M, K, G, has_g_idx)) return 0;
  const int sp = rows_splits(N, K);
  return sp > 1 ? static_cast<size_t>(sp) * static_cast<size_t>(M) * static_cast<size_t>(N) * sizeof(float) : 0;
}

hipError_t launch_linear_skinny(const LinearArgs& a, hipStream_t s) {
  if (!skinny_supported(a)) return hipErrorInvalidValue;
  if (batched_ok(a)) return launch_batched(a, s);
  if (rows_ok(a)) return a.asym ? launch_rows2<true>(a, s) : launch_rows2<false>(a, s);
  // M = 1: the dot-product kernel streams rows fastest; M = 2..4: the
  // matrix-core kernel, whose cost does not grow with M.
  if (a.M >= 2 && mfma_ok(a)) {
    if (a.M == 2) return launch_mfma2<2>(a, s);
    return launch_mfma2<4>(a, s);
  }
  if (stream_ok(a)) return launch_stream(a, s);
  if (act_mma_ok(a)) return launch_act_mma(a, s);
  if (act_ok(a)) return launch_act(a, s);
  if (dot2_ok(a)) {
    if (a.M == 1) return launch_dot2<1>(a, s);
    if (a.M == 2) return launch_dot2<2>(a, s);
    return launch_dot2<4>(a, s);
  }
  if (mfma_ok(a)) return launch_mfma2<1>(a, s);
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
