// Host-side launchers shared between the libw4 translation units.  Arguments
// are validated by the C-ABI layer (w4_api.hip) before any of these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4 {

struct QuantArgs {
  const void* w;
  int w_bf16;           // 0: fp32 weights, 1: bf16 weights
  int64_t N, K, G, NG;
  int asym;             // 0: signed codes, 1: codes with zero-points
  const int32_t* g_idx; // NULL: contiguous groups
  uint8_t* codes;
  float* scales;
  uint8_t* zeros;
};

struct DequantArgs {
  const uint8_t* codes;
  const float* scales;
  const uint8_t* zeros;
  const int32_t* g_idx;
  int64_t N, K, G, NG;
  int asym;
  void* out;
  int out_bf16;         // 0: fp32 output, 1: bf16 output
  int zpk;              // zero-points packed two per byte [N, ceil(NG/2)]
};

struct LinearArgs {
  const uint16_t* x;    // bf16 [M, K]
  int64_t M;
  const uint8_t* codes;
  const float* scales;
  const uint8_t* zeros;
  const int32_t* g_idx;
  int64_t N, K, G, NG;
  int asym;
  const uint16_t* bias; // bf16 [N] or NULL
  uint16_t* y;          // bf16 [M, N]
  float* partial;       // workspace for split-K partial sums (batched decode), or NULL
  int zpk;              // zero-points packed two per byte [N, ceil(NG/2)]
};

struct GradArgs {
  const uint16_t* dy;   // bf16 [M, N]
  int64_t M;
  const uint8_t* codes;
  const float* scales;
  const uint8_t* zeros;
  const int32_t* g_idx;
  int64_t N, K, G, NG;
  int asym;
  uint16_t* dx;         // bf16 [M, K]
  float* partial;       // workspace: fp32 slice partials (M <= 16) or bf16 Wd^T (M > 16)
  int zpk;              // zero-points packed two per byte [N, ceil(NG/2)]
};

// Input-gradient plan: M <= kGradSkinnyMax splits the rows of W into `slices`
// of `rows_per` rows with fp32 partials (at most kGradPartialBytes of them);
// larger M stages Wd^T.  `workspace` is the byte count either needs.
constexpr int64_t kGradSkinnyMax = 16;
constexpr int64_t kGradPartialBytes = int64_t(16) << 20;
struct GradPlan {
  int slices, rows_per;
  size_t workspace;
};
GradPlan grad_plan(int64_t M, int64_t N, int64_t K, int64_t G, bool has_g_idx);
hipError_t launch_grad_input(const GradArgs& a, hipStream_t s);

struct LoraArgs {
  const uint8_t* codes;
  const float* scales;
  const uint8_t* zeros;
  const int32_t* g_idx;
  int64_t N, K, G, NG;
  int asym;
  const float* a;       // fp32 [K, r]
  const float* b;       // fp32 [r, N]
  int r;
  float c;              // scale of the update (alpha / rank)
  uint8_t* codes_out;   // may be `codes` (in place)
  float* scales_out;    // may be `scales`
  uint8_t* zeros_out;   // may be `zeros`
  float* merged;        // workspace: fp32 [N, K] merged weight (generic path)
};

// LoRA merge: contiguous power-of-two groups of 8 .. 512 columns with rank <=
// kLoraMaxRank merge and quantize in one kernel (no workspace); any other
// layout writes the merged fp32 weight to the workspace and quantizes it.
constexpr int kLoraMaxRank = 64;
bool lora_fused(int64_t K, int64_t G, bool has_g_idx, int64_t r);
size_t lora_workspace_bytes(int64_t N, int64_t K, int64_t G, bool has_g_idx, int64_t r);
hipError_t launch_lora_merge(const LoraArgs& a, hipStream_t s);

// Storage formats: GGUF Q4_0 blocks of an [N, K] weight (K % 32 == 0) and
// packed zero-points [N, ceil(NG/2)].
hipError_t launch_q4_0_quantize(const void* w, bool bf16, int64_t N, int64_t K, uint8_t* blocks, hipStream_t s);
hipError_t launch_q4_0_dequantize(const uint8_t* blocks, int64_t N, int64_t K, void* out, bool bf16, hipStream_t s);
hipError_t launch_pack_zeros(const uint8_t* z, int64_t N, int64_t NG, uint8_t* packed, hipStream_t s);
hipError_t launch_unpack_zeros(const uint8_t* packed, int64_t N, int64_t NG, uint8_t* z, hipStream_t s);

// Largest group count the quantizer's per-row LDS tables hold.
constexpr int64_t kMaxGroupsPerRow = 4096;

hipError_t launch_quantize_pack(const QuantArgs& a, hipStream_t s);
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t s);

// Skinny linear (M <= 16).  Returns hipErrorInvalidValue if no skinny kernel
// covers the request (the caller then takes the prefill path).
bool skinny_supported(const LinearArgs& a);
hipError_t launch_linear_skinny(const LinearArgs& a, hipStream_t s);
// The streaming decode GEMV (M = 1, K = 4096, contiguous groups, G % 32 == 0)
// and its rows per row set for N rows (also used by the act-order decode).
bool stream_ok(const LinearArgs& a);
hipError_t launch_stream(const LinearArgs& a, hipStream_t s);
int stream_rows(int64_t N);
// The one-launch batched decode (4 < M <= 16, contiguous groups of 32, 64 or a
// multiple of 128, K % 128 == 0).
bool batched_shape_ok(int64_t N, int64_t M, int64_t K, int64_t G, bool has_g_idx, bool asym);
// The act-order decode on the matrix cores (M = 1, g_idx, at most 32 groups
// per row, K % 1024 == 0).
bool act_mma_ok(const LinearArgs& a);
hipError_t launch_act_mma(const LinearArgs& a, hipStream_t s);
bool batched_ok(const LinearArgs& a);
hipError_t launch_batched(const LinearArgs& a, hipStream_t s);
// Workspace the skinny path needs (fp32 split-K partials of the batched
// decode kernel; 0 when it runs in one pass).
size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G, bool has_g_idx, bool asym);

// Allow `bytes` of dynamic LDS for `kernel` on device `dev` (once per pair,
// thread-safe).
hipError_t ensure_lds_attribute(const void* kernel, int bytes, int dev);

// Fragment-tiled bf16 weight for the prefill GEMM (N % 128 == 0, K % 64 == 0):
// the 8 columns k .. k + 7 (k % 8 == 0) of row n form one 16-byte unit at
// unit index ((nb KT + kt) 4 + ks) 64 + 32 h + rr, where nb = n / 32,
// rr = n % 32, KT = K / 64, kt = k / 64, c = (k % 64) / 8, h = c / 4,
// ks = c % 4.  One MFMA operand fragment of a wave is then 1 KB contiguous.
__host__ __device__ inline int64_t tiled_unit(int64_t n, int64_t k, int64_t K) {
  const int64_t c = (k % 64) / 8;
  return (((n / 32) * (K / 64) + k / 64) * 4 + (c % 4)) * 64 + 32 * (c / 4) + n % 32;
}
bool gemm_tiled_ok(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_tiled(const uint16_t* x, const uint16_t* wt, const uint16_t* bias, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, hipStream_t s);
// Dequantize to the tiled bf16 layout; false when the shape is not covered
// (then the plain row-major dequantize and GEMM run).
bool dequantize_tiled_ok(const DequantArgs& a);
hipError_t launch_dequantize_tiled(const DequantArgs& a, hipStream_t s);

// Dense bf16 GEMM  y = x . wd^T + bias  (x [M, K], wd [N, K], y [M, N]).
hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* wd,
                            const uint16_t* bias, uint16_t* y, int64_t M,
                            int64_t N, int64_t K, hipStream_t s);

}  // namespace w4
