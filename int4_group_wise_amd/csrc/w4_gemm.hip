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
#include <mutex>
#include <set>
#include <type_traits>
#include <utility>

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
  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      const int r = c >> 3, kc = (c & 7) * 8;
      const int gk = k0 + kc;
      const int gm = m0 + r, gn = n0 + r;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      ra[i] = (gm < M && gk < K) ? *reinterpret_cast<const u32x4*>(x + static_cast<int64_t>(gm) * K + gk) : zero;
      rb[i] = (gn < N && gk < K) ? *reinterpret_cast<const u32x4*>(wd + static_cast<int64_t>(gn) * K + gk) : zero;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      const int r = c >> 3, kc = (c & 7) * 8;
      *reinterpret_cast<u32x4*>(&As[r * kLdsStride + kc]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[r * kLdsStride + kc]) = rb[i];
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

// ---------------------------------------------------------------------------
// Pipelined GEMM for K % 64 == 0: 256 x 128 output tile per 256-thread
// workgroup (2 x 2 waves of 128 x 64, i.e. 8 x 4 MFMA tiles of 16 x 16 per
// wave), K stepped by 64 through a 3-stage LDS ring filled by direct
// global -> LDS loads (global_load_lds_dwordx4), so two K-steps are in flight
// while one is consumed without staging registers.
//
// LDS layout of a stage: A rows (256) then B rows (128), 128 bytes each (64
// bf16), split in 8 chunks of 16 bytes; chunk c of row r is stored at slot
// c ^ swz(r).  A 16-byte LDS read serves 16 lanes per cycle from 64 banks (8
// lanes from 32 banks on parts with 32); swz keeps the 16 rows such a group
// touches on distinct 16-byte bank groups either way.  A load instruction
// fills 1 KB of consecutive slots (8 rows): lane i writes slot i, so lane i
// fetches the global chunk that belongs there.
// ---------------------------------------------------------------------------
constexpr int PM = 256, PN = 128, PK = 64, PSTAGES = 3;
constexpr int kPStageBytes = (PM + PN) * PK * 2;          // 48 KB
constexpr int kPLdsBytes = PSTAGES * kPStageBytes;       // 144 KB

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ void lds_dma16(const void* gsrc, void* ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                       reinterpret_cast<uintptr_t>(ldst)), 16, 0, 0);
}

// The same copy through a buffer descriptor (MUBUF with the lds bit): the
// compiler counts it on vmcnt alone, so fragment reads issued while such loads
// are in flight keep exact lgkmcnt waits (with the global form it waits for
// every LDS read), and an offset past the descriptor's size reads zeros.
__device__ __forceinline__ void lds_buf16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* ldst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                               reinterpret_cast<uintptr_t>(ldst)), 16, voff, 0, 0, 0);
}

// Tile (row tile tm, column tile tn) of workgroup b.  Workgroups are dealt to
// the 8 XCDs round-robin (b % 8) and each XCD has its own L2, so when the tile
// count divides by 8 each XCD's share is made a contiguous run of positions,
// and positions are walked in groups of 4 row tiles across all column tiles:
// on a 8 x 32 tile grid every XCD takes a 4 x 8 block (16 MB of operands per
// L2 instead of 20 MB with row-major order; the GEMM 84.5 -> 83.2 us).
__device__ __forceinline__ void pipe_tile(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nt = tiles_m * tiles_n;
  const int p = nt % 8 == 0 ? (b % 8) * (nt / 8) + b / 8 : b;
  constexpr int kGroupM = 4;
  const int gsz = kGroupM * tiles_n;
  const int first = (p / gsz) * kGroupM;
  const int rows = min(kGroupM, tiles_m - first);
  const int r = p % gsz;
  tm = first + r % rows;
  tn = r / rows;
}

__global__ __launch_bounds__(kThreads) void gemm_bf16_pipe_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wd,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int M, int N, int K) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t psm[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 1, wn = wid & 1;
  const int tiles_n = (N + PN - 1) / PN;
  int tm, tn;
  pipe_tile(blockIdx.x, (M + PM - 1) / PM, tiles_n, tm, tn);
  const int m0 = tm * PM;
  const int n0 = tn * PN;

  // loads: wave wid fills A rows [64 wid, 64 wid + 64) (8 instructions of 8
  // rows) and B rows [32 wid, 32 wid + 32) (4 instructions); lane i of an
  // instruction covering rows r0..r0+7 writes slot i = (row r0 + i / 8,
  // slot i % 8) and fetches chunk (i % 8) ^ (row & 7) of that row.  Rows past
  // M or N fetch a valid row instead: their outputs are never stored.
  const int lr = lane >> 3, ls = lane & 7;
  const uint16_t* asrc[8];
  const uint16_t* bsrc[4];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = 64 * wid + 8 * p + lr;
    const int gm = min(m0 + r, M - 1);
    asrc[p] = x + static_cast<int64_t>(gm) * K + 8 * (ls ^ swz(r));
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = 32 * wid + 8 * p + lr;
    const int gn = min(n0 + r, N - 1);
    bsrc[p] = wd + static_cast<int64_t>(gn) * K + 8 * (ls ^ swz(r));
  }
  auto issue = [&](int kt) {
    uint8_t* st = psm + (kt % PSTAGES) * kPStageBytes;
    const int k0 = kt * PK;
#pragma unroll
    for (int p = 0; p < 8; ++p) lds_dma16(asrc[p] + k0, st + (64 * wid + 8 * p) * 128);
#pragma unroll
    for (int p = 0; p < 4; ++p) lds_dma16(bsrc[p] + k0, st + PM * 128 + (32 * wid + 8 * p) * 128);
  };

  // wave tile 128 x 64 = 4 x 2 tiles of 32 x 32 (v_mfma_f32_32x32x16_bf16,
  // which sustains a higher rate than 16 x 16 x 32 with one wave per SIMD)
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = K / PK;
  issue(0);
  if (nk > 1) issue(1);
  const int fr = lane & 31, fh = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    // this thread's loads of stage kt are done once at most the next stage's
    // 12 loads are outstanding; the barrier then covers every thread's
    // s_waitcnt encodes vmcnt in bits 3:0 and 15:14, lgkmcnt in 11:8, expcnt
    // in 6:4; 0x0F7C = vmcnt(12), 0x0F70 = vmcnt(0), the others not waited on.
    if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(0x0F7C);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    // a bare barrier: __syncthreads would also wait for the next stage's
    // loads.  The empty asm keeps the compiler from moving LDS reads across.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 2 < nk) issue(kt + 2);
    const uint8_t* st = psm + (kt % PSTAGES) * kPStageBytes;
    const uint8_t* sa = st + (wm * 128) * 128;
    const uint8_t* sb = st + PM * 128 + (wn * 64) * 128;
    // Fragments of all four 16-column sub-steps are read up front, so later
    // sub-steps' reads are in flight while earlier MFMAs run.  32 x 32 x 16
    // operand layout: lane l holds row (or column) l % 32, k = 8 (l / 32) + e.
    bf16x8_t af[4][4], bfr[4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int chunk = 2 * ks + fh;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 32 * j + fr;
        bfr[ks][j] = *reinterpret_cast<const bf16x8_t*>(sb + r * 128 + 16 * (chunk ^ swz(r)));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 32 * i + fr;
        af[ks][i] = *reinterpret_cast<const bf16x8_t*>(sa + r * 128 + 16 * (chunk ^ swz(r)));
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
  }

  // 32 x 32 accumulator layout: register v of lane l holds row
  // 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + fr;
    if (n >= N) continue;
    const float b = bias ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 128 + i * 32 + 8 * (v / 4) + 4 * fh + (v % 4);
        if (m < M) y[static_cast<int64_t>(m) * N + n] = static_cast<uint16_t>(f32_to_bf16(acc[i][j][v] + b));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// GEMM with a fragment-tiled weight (N % 128 == 0, K % 64 == 0): the same
// 256 x 128 x 64 workgroup tile, 2 x 2 waves of 128 x 64 and
// v_mfma_f32_32x32x16_bf16 as gemm_bf16_pipe_kernel, but only the activation
// tile goes through LDS (a 4-stage ring of 32 KB stages filled by direct
// buffer loads).  The weight comes from the tiled layout written by the
// dequantizer (w4_internal.h, tiled_unit): every 16-byte piece a lane needs for
// one MFMA sits at consecutive addresses across the wave, so a wave reads its
// weight fragments with fully coalesced 1 KB loads straight into registers.
// Both are issued three K-steps ahead: the operands come from the L2 or past
// it, and with one wave per SIMD nothing else hides their latency (two steps
// ahead took 2.5 us more per call at the prefill shape, four 1 us less).  Per
// K-step a CU moves 32 KB of direct-load writes and 64 KB of fragment reads
// through LDS instead of 48 KB and 96 KB.
//
// K order inside a K-step: lane half h of an MFMA operand holds columns
// 32 h + 8 ks .. 32 h + 8 ks + 7 for MFMA ks (activations: LDS chunk 4 h + ks
// of the row; weight: the tiled unit (ks, h)); both operands agree, so the
// MFMA sums the same products as with the natural order.
// ---------------------------------------------------------------------------
constexpr int TM = 256, TN = 128, TK = 64, TSTAGES = 4;
constexpr int kTStageBytes = TM * TK * 2;                // 32 KB: activations only
constexpr int kTLdsBytes = TSTAGES * kTStageBytes;       // 128 KB

__global__ __launch_bounds__(kThreads) void gemm_tiled_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wt,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int M, int N, int K) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t tsm[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 1, wn = wid & 1;
  const int tiles_n = N / TN;
  int tm, tn;
  pipe_tile(blockIdx.x, (M + TM - 1) / TM, tiles_n, tm, tn);
  const int m0 = tm * TM;
  const int n0 = tn * TN;
  const int KT = K / TK;

  // activation loads: as in gemm_bf16_pipe_kernel (wave wid fills rows
  // [64 wid, 64 wid + 64), lane i of an 8-row instruction slot i)
  const int lr = lane >> 3, ls = lane & 7;
  // byte offsets from x (the launcher checks that x fits in 31 bits)
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x), 0, M * K * 2, 0x00020000);
  uint32_t aoff[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = 64 * wid + 8 * p + lr;
    const int gm = min(m0 + r, M - 1);    // rows past M load a valid row; never stored
    aoff[p] = (static_cast<uint32_t>(gm) * static_cast<uint32_t>(K) + 8u * (ls ^ swz(r))) * 2u;
  }
  // weight: this wave's two 32-row blocks; unit (nb, kt, ks) starts at
  // ((nb KT + kt) 4 + ks) 64 units of 8 bf16, lane l at + l
  const int nb0 = (n0 + 64 * wn) / 32;
  const uint16_t* bsrc0 = wt + (static_cast<int64_t>(nb0) * KT * 4 * 64 + lane) * 8;
  const int64_t bstride_nb = static_cast<int64_t>(KT) * 4 * 64 * 8;   // bf16 per 32-row block
  u32x4 breg[TSTAGES][2][4];

  // loads of K-step kt into stage S, half H: activation instruction slots
  // 4H .. 4H + 3 and the weight block j = H
  auto issue_half = [&](auto stage, auto half, int kt) {
    constexpr int S = decltype(stage)::value;
    constexpr int H = decltype(half)::value;
    uint8_t* st = tsm + S * kTStageBytes;
    const int k0 = kt * TK;
#pragma unroll
    for (int p = 4 * H; p < 4 * H + 4; ++p) lds_buf16(xr, aoff[p] + 2u * k0, st + (64 * wid + 8 * p) * 128);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      breg[S][H][ks] = *reinterpret_cast<const u32x4*>(bsrc0 + H * bstride_nb + (static_cast<int64_t>(kt) * 4 + ks) * 512);
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int fr = lane & 31, fh = lane >> 5;
  bf16x8_t af[4][4];   // [k-slice][row block] activation fragments
  auto read_frag = [&](auto stage, auto slice) {
    constexpr int S = decltype(stage)::value;
    constexpr int KS = decltype(slice)::value;
    const uint8_t* sa = tsm + S * kTStageBytes + (wm * 128) * 128;
    const int chunk = 4 * fh + KS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * i + fr;
      af[KS][i] = *reinterpret_cast<const bf16x8_t*>(sa + r * 128 + 16 * (chunk ^ swz(r)));
    }
  };
  auto mma = [&](auto stage, int ks) {
    constexpr int S = decltype(stage)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            af[ks][i], __builtin_bit_cast(bf16x8_t, breg[S][j][ks]), acc[i][j], 0, 0, 0);
  };
  // one half-step's order: the 8 fragment reads spread over its first 8
  // MFMAs, the 8 loads over all 16
  auto order = [&]() {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  };

  // K-step kt (stage S): the first half runs the MFMAs of k-slices 0 and 1
  // (fragments read during the previous step) while it reads slices 2 and 3;
  // then, once every wave's loads of stage S + 1 have landed (one barrier per
  // step), the second half runs slices 2 and 3 while it reads slices 0 and 1
  // of stage S + 1.  Both halves issue half of the loads of step kt + 3 (the
  // last steps' clamped to step KT - 1 again: the stage they fill is no longer
  // read), so the count of loads in flight is the same at every barrier: 8 of
  // step kt + 3 after the 16 each of steps kt + 1 and kt + 2.  The stage those
  // loads fill was last read in step kt - 1, whose reads every wave finished
  // before the barrier of step kt - 1 (lgkmcnt(0) there).
  auto step = [&](auto stage, int kt) {
    constexpr int S = decltype(stage)::value;
    constexpr int SN = (S + 1) % TSTAGES;
    constexpr int SL = (S + 3) % TSTAGES;
    const int kl = min(kt + 3, KT - 1);
    issue_half(std::integral_constant<int, SL>{}, std::integral_constant<int, 0>{}, kl);
    read_frag(std::integral_constant<int, S>{}, std::integral_constant<int, 2>{});
    read_frag(std::integral_constant<int, S>{}, std::integral_constant<int, 3>{});
    mma(std::integral_constant<int, S>{}, 0);
    mma(std::integral_constant<int, S>{}, 1);
    order();
    __builtin_amdgcn_sched_barrier(0);
    // s_waitcnt: vmcnt in bits 3:0 and 15:14, lgkmcnt in 11:8, expcnt in 6:4;
    // 0x4078 = vmcnt(24) lgkmcnt(0)
    __builtin_amdgcn_s_waitcnt(0x4078);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue_half(std::integral_constant<int, SL>{}, std::integral_constant<int, 1>{}, kl);
    read_frag(std::integral_constant<int, SN>{}, std::integral_constant<int, 0>{});
    read_frag(std::integral_constant<int, SN>{}, std::integral_constant<int, 1>{});
    mma(std::integral_constant<int, S>{}, 2);
    mma(std::integral_constant<int, S>{}, 3);
    order();
    __builtin_amdgcn_sched_barrier(0);
  };

  issue_half(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, 0);
  issue_half(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, 0);
  issue_half(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{}, min(1, KT - 1));
  issue_half(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}, min(1, KT - 1));
  issue_half(std::integral_constant<int, 2>{}, std::integral_constant<int, 0>{}, min(2, KT - 1));
  issue_half(std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{}, min(2, KT - 1));
  // stage 0 landed in every wave (0x8F70 = vmcnt(32)); its slices 0 and 1
  __builtin_amdgcn_s_waitcnt(0x8F70);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read_frag(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
  read_frag(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
  __builtin_amdgcn_sched_barrier(0);
  int kt = 0;
  for (; kt + TSTAGES <= KT; kt += TSTAGES) {
    step(std::integral_constant<int, 0>{}, kt);
    step(std::integral_constant<int, 1>{}, kt + 1);
    step(std::integral_constant<int, 2>{}, kt + 2);
    step(std::integral_constant<int, 3>{}, kt + 3);
  }
  if (kt < KT) step(std::integral_constant<int, 0>{}, kt);
  if (kt + 1 < KT) step(std::integral_constant<int, 1>{}, kt + 1);
  if (kt + 2 < KT) step(std::integral_constant<int, 2>{}, kt + 2);
  // the direct loads of the last issues must land before the workgroup's LDS
  // is released (0x0F70 = vmcnt(0))
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // 32 x 32 accumulator layout: register v of lane l holds row
  // 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + fr;
    const float b = bias ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 128 + i * 32 + 8 * (v / 4) + 4 * fh + (v % 4);
        if (m < M) y[static_cast<int64_t>(m) * N + n] = static_cast<uint16_t>(f32_to_bf16(acc[i][j][v] + b));
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

// Dynamic LDS above the default limit must be allowed per kernel; the call is
// made once per (kernel, device) and remembered under a lock.
hipError_t ensure_lds_attribute(const void* kernel, int bytes, int dev) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kernel, dev})) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({kernel, dev});
  return e;
}


bool gemm_tiled_ok(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && N % TN == 0 && K % TK == 0 && M * K * 2 < (int64_t{1} << 31) && N <= INT32_MAX && K <= INT32_MAX;
}

hipError_t launch_gemm_tiled(const uint16_t* x, const uint16_t* wt, const uint16_t* bias, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = ensure_lds_attribute(reinterpret_cast<const void*>(gemm_tiled_kernel), kTLdsBytes, dev);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((M + TM - 1) / TM) * (N / TN);
  gemm_tiled_kernel<<<dim3(static_cast<uint32_t>(tiles)), dim3(kThreads), kTLdsBytes, s>>>(
      x, wt, bias, y, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* wd, const uint16_t* bias,
                            uint16_t* y, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  if (K % PK == 0 && M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = ensure_lds_attribute(reinterpret_cast<const void*>(gemm_bf16_pipe_kernel), kPLdsBytes, dev);   // the 144 KB ring
    if (e != hipSuccess) return e;
    const int64_t tiles = ((M + PM - 1) / PM) * ((N + PN - 1) / PN);
    gemm_bf16_pipe_kernel<<<dim3(static_cast<uint32_t>(tiles)), dim3(kThreads), kPLdsBytes, s>>>(
        x, wd, bias, y, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
  } else if (K % 8 == 0 && M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX) {
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
