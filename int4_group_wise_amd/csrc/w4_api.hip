// C ABI of libw4.so (declared in include/w4.h): host-side argument checks and
// dispatch to the gfx950 kernels.  Nothing here allocates device memory.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "w4.h"
#include "w4_internal.h"

namespace {

thread_local std::string g_last_error;

w4_status fail(w4_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

w4_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return W4_OK;
  return fail(W4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxDim = int64_t(1) << 30;       // per-dimension limit (32-bit index math)
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

// Checks shared by the three compute entry points.
w4_status check_format(int64_t N, int64_t K, int64_t G, int mode, const void* zeros,
                       const void* g_idx, const char* fn) {
  if (N < 1 || K < 1) return fail(W4_ERR_INVALID_ARG, "%s: N and K must be >= 1 (got N=%lld K=%lld)", fn, (long long)N, (long long)K);
  if (N > kMaxDim || K > kMaxDim) return fail(W4_ERR_UNSUPPORTED, "%s: N and K must be <= 2^30", fn);
  if (G != W4_PER_CHANNEL && G < K && (G < 8 || G % 8 != 0))
    return fail(W4_ERR_INVALID_ARG, "%s: group size G must be a multiple of 8 (>= 8), >= K, or W4_PER_CHANNEL (got %lld)",
                fn, (long long)G);
  if (mode != W4_SYM && mode != W4_ASYM && mode != W4_ASYM_PACKED)
    return fail(W4_ERR_INVALID_ARG, "%s: mode must be W4_SYM, W4_ASYM or W4_ASYM_PACKED", fn);
  if (mode != W4_SYM && zeros == nullptr) return fail(W4_ERR_INVALID_ARG, "%s: zero-point modes need zero-points", fn);
  if (mode == W4_SYM && zeros != nullptr) return fail(W4_ERR_INVALID_ARG, "%s: W4_SYM takes no zero-points (pass NULL)", fn);
  if (zeros && !aligned16(zeros)) return fail(W4_ERR_INVALID_ARG, "%s: zeros must be 16-byte aligned", fn);
  if (g_idx && !aligned16(g_idx)) return fail(W4_ERR_INVALID_ARG, "%s: g_idx must be 16-byte aligned", fn);
  return W4_OK;
}

// Group size as the kernels take it.  W4_PER_CHANNEL or G >= K is one group
// per row; every multiple of 128 that is >= K maps all columns to group 0 and
// keeps open the fast paths that require G % 128 == 0.
int64_t kernel_group(int64_t K, int64_t G) {
  if (G == W4_PER_CHANNEL || G >= K) return (K + 127) / 128 * 128;
  return G;
}

}  // namespace

extern "C" {

int w4_abi_version(void) { return W4_ABI_VERSION; }

const char* w4_status_string(int status) {
  switch (status) {
    case W4_OK: return "ok";
    case W4_ERR_INVALID_ARG: return "invalid argument";
    case W4_ERR_UNSUPPORTED: return "unsupported";
    case W4_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* w4_last_error(void) { return g_last_error.c_str(); }

w4_status w4_quantize_pack(const void* w, int w_dtype, int64_t N, int64_t K, int64_t G, int mode,
                           const int32_t* g_idx, uint8_t* codes, float* scales, uint8_t* zeros,
                           void* stream) {
  g_last_error.clear();
  const char* fn = "w4_quantize_pack";
  if (w4_status st = check_format(N, K, G, mode, zeros, g_idx, fn)) return st;
  if (mode == W4_ASYM_PACKED)
    return fail(W4_ERR_UNSUPPORTED, "%s: writes one zero-point per byte (W4_ASYM); pack them with w4_pack_zeros", fn);
  G = kernel_group(K, G);
  if (w_dtype != W4_F32 && w_dtype != W4_BF16) return fail(W4_ERR_INVALID_ARG, "%s: w_dtype must be W4_F32 or W4_BF16", fn);
  if (!w || !codes || !scales) return fail(W4_ERR_INVALID_ARG, "%s: w, codes and scales must be non-NULL", fn);
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales))
    return fail(W4_ERR_INVALID_ARG, "%s: w, codes and scales must be 16-byte aligned", fn);
  const int64_t NG = (K + G - 1) / G;
  if (NG > w4::kMaxGroupsPerRow)
    return fail(W4_ERR_UNSUPPORTED, "%s: at most %lld groups per row (got %lld)", fn, (long long)w4::kMaxGroupsPerRow, (long long)NG);
  if (N > kMaxGrid) return fail(W4_ERR_UNSUPPORTED, "%s: too many rows", fn);
  w4::QuantArgs a{w, w_dtype == W4_BF16, N, K, G, NG, mode == W4_ASYM, g_idx, codes, scales, zeros};
  return hip_status(w4::launch_quantize_pack(a, static_cast<hipStream_t>(stream)), fn);
}

w4_status w4_dequantize(const uint8_t* codes, const float* scales, const uint8_t* zeros,
                        const int32_t* g_idx, int64_t N, int64_t K, int64_t G, int mode,
                        void* out, int out_dtype, void* stream) {
  g_last_error.clear();
  const char* fn = "w4_dequantize";
  if (w4_status st = check_format(N, K, G, mode, zeros, g_idx, fn)) return st;
  G = kernel_group(K, G);
  if (out_dtype != W4_F32 && out_dtype != W4_BF16) return fail(W4_ERR_INVALID_ARG, "%s: out_dtype must be W4_F32 or W4_BF16", fn);
  if (!codes || !scales || !out) return fail(W4_ERR_INVALID_ARG, "%s: codes, scales and out must be non-NULL", fn);
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(out))
    return fail(W4_ERR_INVALID_ARG, "%s: codes, scales and out must be 16-byte aligned", fn);
  const int64_t NG = (K + G - 1) / G;
  const int64_t chunk_blocks = ((K + 7) / 8 + 255) / 256;
  if (N * chunk_blocks > kMaxGrid) return fail(W4_ERR_UNSUPPORTED, "%s: matrix too large for one launch", fn);
  w4::DequantArgs a{codes, scales, zeros, g_idx, N, K, G, NG, mode != W4_SYM, out, out_dtype == W4_BF16,
                    mode == W4_ASYM_PACKED};
  return hip_status(w4::launch_dequantize(a, static_cast<hipStream_t>(stream)), fn);
}

size_t w4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G, int mode, int has_g_idx) {
  if (M < 1 || N < 1 || K < 1 || (G < 1 && G != W4_PER_CHANNEL)) return 0;
  if (M <= 16)   // fp32 split-K partials of the K-split batched decode kernel, if it is the one that runs
    return w4::skinny_workspace_bytes(M, N, K, kernel_group(K, G), has_g_idx != 0, mode != W4_SYM);
  return static_cast<size_t>(N) * static_cast<size_t>(K) * 2u;   // bf16 dequantized weight
}

}  // extern "C"

namespace {

// The body of w4_linear; `fn` names the entry point in error messages.
w4_status linear_impl(const void* x, int64_t M, const uint8_t* codes, const float* scales,
                      const uint8_t* zeros, const int32_t* g_idx, int64_t N, int64_t K, int64_t G,
                      int mode, const void* bias, void* y, void* workspace, size_t workspace_bytes,
                      void* stream, const char* fn) {
  if (w4_status st = check_format(N, K, G, mode, zeros, g_idx, fn)) return st;
  G = kernel_group(K, G);
  if (M < 0) return fail(W4_ERR_INVALID_ARG, "%s: M must be >= 0", fn);
  if (M > kMaxDim) return fail(W4_ERR_UNSUPPORTED, "%s: M must be <= 2^30", fn);
  if (M == 0) return W4_OK;
  if (!x || !codes || !scales || !y) return fail(W4_ERR_INVALID_ARG, "%s: x, codes, scales and y must be non-NULL", fn);
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned16(y) || (bias && !aligned16(bias)))
    return fail(W4_ERR_INVALID_ARG, "%s: x, codes, scales, bias and y must be 16-byte aligned", fn);
  const int64_t NG = (K + G - 1) / G;
  hipStream_t s = static_cast<hipStream_t>(stream);
  w4::LinearArgs a{static_cast<const uint16_t*>(x), M, codes, scales, zeros, g_idx, N, K, G, NG,
                   mode != W4_SYM, static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), nullptr,
                   mode == W4_ASYM_PACKED};
  const size_t need = w4_linear_workspace_bytes(M, N, K, G, mode, g_idx != nullptr);
  if (workspace_bytes < need || (need && !workspace))
    return fail(W4_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  if (need && !aligned16(workspace)) return fail(W4_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
  if (w4::skinny_supported(a)) {
    a.partial = need ? static_cast<float*>(workspace) : nullptr;
    return hip_status(w4::launch_linear_skinny(a, s), fn);
  }
  const int64_t chunk_blocks = ((K + 7) / 8 + 255) / 256;
  const int64_t gemm_blocks = K % 8 == 0 ? ((M + 127) / 128) * ((N + 127) / 128) : (M * N + 255) / 256;
  if (N * chunk_blocks > kMaxGrid || gemm_blocks > kMaxGrid)
    return fail(W4_ERR_UNSUPPORTED, "%s: matrix too large for one launch", fn);
  w4::DequantArgs d{codes, scales, zeros, g_idx, N, K, G, NG, mode != W4_SYM, workspace, 1, mode == W4_ASYM_PACKED};
  if (w4::gemm_tiled_ok(M, N, K) && w4::dequantize_tiled_ok(d)) {
    // the weight dequantized into the GEMM's fragment-tiled layout
    if (w4_status st = hip_status(w4::launch_dequantize_tiled(d, s), fn)) return st;
    return hip_status(w4::launch_gemm_tiled(a.x, static_cast<const uint16_t*>(workspace), a.bias, a.y, M, N, K, s), fn);
  }
  if (w4_status st = hip_status(w4::launch_dequantize(d, s), fn)) return st;
  return hip_status(w4::launch_gemm_bf16(a.x, static_cast<const uint16_t*>(workspace), a.bias, a.y, M, N, K, s), fn);
}

// Scratch of w4_linear_noalloc: device memory of fixed size that every GPU
// the library runs on holds until the process ends.  Host code uses the
// per-device address from hipGetSymbolAddress, never the array's name.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's scratch address, looked up once per device with that device
// current.
w4_status scratch_address(void** out, const char* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(W4_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    if (!p) return fail(W4_ERR_HIP, "%s: no device address for the scratch array", fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return W4_OK;
}

}  // namespace

extern "C" {

size_t w4_linear_noalloc_max_scratch_bytes(void) { return kNoAllocScratchBytes; }

w4_status w4_linear_noalloc(const void* x, int64_t M, const uint8_t* codes, const float* scales,
                            const uint8_t* zeros, const int32_t* g_idx, int64_t N, int64_t K, int64_t G,
                            int mode, const void* bias, void* y, void* stream) {
  g_last_error.clear();
  const char* fn = "w4_linear_noalloc";
  if (M > 0 && N >= 1 && K >= 1 && (G >= 1 || G == W4_PER_CHANNEL)) {
    const size_t need = w4_linear_workspace_bytes(M, N, K, G, mode, g_idx != nullptr);
    if (need > kNoAllocScratchBytes)
      return fail(W4_ERR_UNSUPPORTED, "%s: this shape needs %zu bytes of scratch, more than the %zu this entry point holds",
                  fn, need, kNoAllocScratchBytes);
    if (need) {
      void* ws = nullptr;
      if (w4_status st = scratch_address(&ws, fn)) return st;
      return linear_impl(x, M, codes, scales, zeros, g_idx, N, K, G, mode, bias, y, ws, kNoAllocScratchBytes,
                         stream, fn);
    }
  }
  return linear_impl(x, M, codes, scales, zeros, g_idx, N, K, G, mode, bias, y, nullptr, 0, stream, fn);
}

w4_status w4_linear(const void* x, int64_t M, const uint8_t* codes, const float* scales,
                    const uint8_t* zeros, const int32_t* g_idx, int64_t N, int64_t K, int64_t G,
                    int mode, const void* bias, void* y, void* workspace, size_t workspace_bytes,
                    void* stream) {
  g_last_error.clear();
  return linear_impl(x, M, codes, scales, zeros, g_idx, N, K, G, mode, bias, y, workspace, workspace_bytes,
                     stream, "w4_linear");
}

size_t w4_linear_grad_input_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t G, int mode,
                                            int has_g_idx) {
  (void)mode;
  if (M < 1 || N < 1 || K < 1 || (G < 1 && G != W4_PER_CHANNEL)) return 0;
  G = kernel_group(K, G);
  return w4::grad_plan(M, N, K, G, has_g_idx != 0).workspace;
}

w4_status w4_linear_grad_input(const void* dy, int64_t M, const uint8_t* codes, const float* scales,
                               const uint8_t* zeros, const int32_t* g_idx, int64_t N, int64_t K,
                               int64_t G, int mode, void* dx, void* workspace, size_t workspace_bytes,
                               void* stream) {
  g_last_error.clear();
  const char* fn = "w4_linear_grad_input";
  if (w4_status st = check_format(N, K, G, mode, zeros, g_idx, fn)) return st;
  G = kernel_group(K, G);
  if (M < 0) return fail(W4_ERR_INVALID_ARG, "%s: M must be >= 0", fn);
  if (M > kMaxDim) return fail(W4_ERR_UNSUPPORTED, "%s: M must be <= 2^30", fn);
  if (M == 0) return W4_OK;
  if (!dy || !codes || !scales || !dx) return fail(W4_ERR_INVALID_ARG, "%s: dy, codes, scales and dx must be non-NULL", fn);
  if (!aligned16(dy) || !aligned16(codes) || !aligned16(scales) || !aligned16(dx))
    return fail(W4_ERR_INVALID_ARG, "%s: dy, codes, scales and dx must be 16-byte aligned", fn);
  const size_t need = w4_linear_grad_input_workspace_bytes(M, N, K, G, mode, g_idx != nullptr);
  if (workspace_bytes < need || !workspace)
    return fail(W4_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  if (!aligned16(workspace)) return fail(W4_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
  const w4::GradPlan plan = w4::grad_plan(M, N, K, G, g_idx != nullptr);
  if (M <= w4::kGradSkinnyMax) {
    const int64_t cb = ((K + 7) / 8 + 255) / 256;
    if (cb > kMaxGrid || plan.slices > 65535 || (M * K + 255) / 256 > kMaxGrid)
      return fail(W4_ERR_UNSUPPORTED, "%s: matrix too large for one launch", fn);
  } else {
    const int64_t gemm_blocks = N % 8 == 0 ? ((M + 127) / 128) * ((K + 127) / 128) : (M * K + 255) / 256;
    if ((K + 63) / 64 > kMaxGrid || (N + 63) / 64 > 65535 || gemm_blocks > kMaxGrid)
      return fail(W4_ERR_UNSUPPORTED, "%s: matrix too large for one launch", fn);
  }
  const int64_t NG = (K + G - 1) / G;
  w4::GradArgs a{static_cast<const uint16_t*>(dy), M, codes, scales, zeros, g_idx, N, K, G, NG,
                 mode != W4_SYM, static_cast<uint16_t*>(dx), static_cast<float*>(workspace), mode == W4_ASYM_PACKED};
  return hip_status(w4::launch_grad_input(a, static_cast<hipStream_t>(stream)), fn);
}

size_t w4_lora_merge_workspace_bytes(int64_t N, int64_t K, int64_t G, int mode, int has_g_idx, int64_t rank) {
  (void)mode;
  if (N < 1 || K < 1 || (G < 1 && G != W4_PER_CHANNEL) || rank < 1) return 0;
  return w4::lora_workspace_bytes(N, K, kernel_group(K, G), has_g_idx != 0, rank);
}

w4_status w4_lora_merge(const uint8_t* codes, const float* scales, const uint8_t* zeros,
                        const int32_t* g_idx, int64_t N, int64_t K, int64_t G, int mode,
                        const float* lora_a, const float* lora_b, int64_t rank, float lora_scale,
                        uint8_t* codes_out, float* scales_out, uint8_t* zeros_out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  const char* fn = "w4_lora_merge";
  if (w4_status st = check_format(N, K, G, mode, zeros, g_idx, fn)) return st;
  if (mode == W4_ASYM_PACKED)
    return fail(W4_ERR_UNSUPPORTED, "%s: takes one zero-point per byte (W4_ASYM); unpack them with w4_unpack_zeros", fn);
  const int64_t Gk = kernel_group(K, G);
  if (rank < 1) return fail(W4_ERR_INVALID_ARG, "%s: rank must be >= 1", fn);
  if (rank > w4::kLoraMaxRank) return fail(W4_ERR_UNSUPPORTED, "%s: rank must be <= %d", fn, w4::kLoraMaxRank);
  if (!codes || !scales || !lora_a || !lora_b || !codes_out || !scales_out)
    return fail(W4_ERR_INVALID_ARG, "%s: codes, scales, lora_a, lora_b, codes_out and scales_out must be non-NULL", fn);
  if ((mode == W4_ASYM) != (zeros_out != nullptr))
    return fail(W4_ERR_INVALID_ARG, "%s: zeros_out must be given for W4_ASYM and NULL for W4_SYM", fn);
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(lora_a) || !aligned16(lora_b) || !aligned16(codes_out) ||
      !aligned16(scales_out) || (zeros_out && !aligned16(zeros_out)))
    return fail(W4_ERR_INVALID_ARG, "%s: every tensor must be 16-byte aligned", fn);
  const int64_t NG = (K + Gk - 1) / Gk;
  if (NG > w4::kMaxGroupsPerRow)
    return fail(W4_ERR_UNSUPPORTED, "%s: at most %lld groups per row (got %lld)", fn, (long long)w4::kMaxGroupsPerRow, (long long)NG);
  // an output is either its input (in place) or disjoint from every input
  const size_t cbytes = static_cast<size_t>(N) * static_cast<size_t>((K + 1) / 2);
  const size_t sbytes = static_cast<size_t>(N) * static_cast<size_t>(NG) * 4u;
  const size_t zbytes = static_cast<size_t>(N) * static_cast<size_t>(NG);
  struct Span { const void* p; size_t n; };
  const Span ins[] = {{codes, cbytes}, {scales, sbytes}, {zeros, zeros ? zbytes : 0}};
  const Span outs[] = {{codes_out, cbytes}, {scales_out, sbytes}, {zeros_out, zeros_out ? zbytes : 0}};
  for (int o = 0; o < 3; ++o)
    for (int i = 0; i < 3; ++i) {
      if (!outs[o].n || !ins[i].n || (o == i && outs[o].p == ins[i].p)) continue;
      const uintptr_t a0 = reinterpret_cast<uintptr_t>(outs[o].p), b0 = reinterpret_cast<uintptr_t>(ins[i].p);
      if (a0 < b0 + ins[i].n && b0 < a0 + outs[o].n)
        return fail(W4_ERR_INVALID_ARG, "%s: an output overlaps an input other than its own", fn);
    }
  const size_t need = w4::lora_workspace_bytes(N, K, Gk, g_idx != nullptr, rank);
  if (workspace_bytes < need || (need && !workspace))
    return fail(W4_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  if (need && !aligned16(workspace)) return fail(W4_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
  if (N > kMaxGrid) return fail(W4_ERR_UNSUPPORTED, "%s: too many rows", fn);
  w4::LoraArgs a{codes, scales, zeros, g_idx, N, K, Gk, NG, mode == W4_ASYM, lora_a, lora_b,
                 static_cast<int>(rank), lora_scale, codes_out, scales_out, zeros_out,
                 static_cast<float*>(workspace)};
  return hip_status(w4::launch_lora_merge(a, static_cast<hipStream_t>(stream)), fn);
}

w4_status w4_pack_zeros(const uint8_t* zeros, int64_t N, int64_t NG, uint8_t* packed, void* stream) {
  g_last_error.clear();
  const char* fn = "w4_pack_zeros";
  if (N < 1 || NG < 1) return fail(W4_ERR_INVALID_ARG, "%s: N and NG must be >= 1", fn);
  if (N > kMaxDim || NG > kMaxDim) return fail(W4_ERR_UNSUPPORTED, "%s: N and NG must be <= 2^30", fn);
  if (!zeros || !packed) return fail(W4_ERR_INVALID_ARG, "%s: zeros and packed must be non-NULL", fn);
  return hip_status(w4::launch_pack_zeros(zeros, N, NG, packed, static_cast<hipStream_t>(stream)), fn);
}

w4_status w4_unpack_zeros(const uint8_t* packed, int64_t N, int64_t NG, uint8_t* zeros, void* stream) {
  g_last_error.clear();
  const char* fn = "w4_unpack_zeros";
  if (N < 1 || NG < 1) return fail(W4_ERR_INVALID_ARG, "%s: N and NG must be >= 1", fn);
  if (N > kMaxDim || NG > kMaxDim) return fail(W4_ERR_UNSUPPORTED, "%s: N and NG must be <= 2^30", fn);
  if (!zeros || !packed) return fail(W4_ERR_INVALID_ARG, "%s: zeros and packed must be non-NULL", fn);
  return hip_status(w4::launch_unpack_zeros(packed, N, NG, zeros, static_cast<hipStream_t>(stream)), fn);
}

namespace {
w4_status check_q4_0(int64_t N, int64_t K, const void* a, const void* b, const char* fn) {
  if (N < 1 || K < 32 || K % 32 != 0)
    return fail(W4_ERR_INVALID_ARG, "%s: N must be >= 1 and K a positive multiple of 32 (got N=%lld K=%lld)", fn,
                (long long)N, (long long)K);
  if (N > kMaxDim || K > kMaxDim) return fail(W4_ERR_UNSUPPORTED, "%s: N and K must be <= 2^30", fn);
  if (!a || !b) return fail(W4_ERR_INVALID_ARG, "%s: pointers must be non-NULL", fn);
  if (!aligned16(a) || !aligned16(b)) return fail(W4_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  if ((N * (K / 32) + 31) / 32 > kMaxGrid) return fail(W4_ERR_UNSUPPORTED, "%s: matrix too large for one launch", fn);
  return W4_OK;
}
}  // namespace

w4_status w4_q4_0_quantize(const void* w, int w_dtype, int64_t N, int64_t K, uint8_t* blocks, void* stream) {
  g_last_error.clear();
  const char* fn = "w4_q4_0_quantize";
  if (w4_status st = check_q4_0(N, K, w, blocks, fn)) return st;
  if (w_dtype != W4_F32 && w_dtype != W4_BF16) return fail(W4_ERR_INVALID_ARG, "%s: w_dtype must be W4_F32 or W4_BF16", fn);
  return hip_status(w4::launch_q4_0_quantize(w, w_dtype == W4_BF16, N, K, blocks, static_cast<hipStream_t>(stream)), fn);
}

w4_status w4_q4_0_dequantize(const uint8_t* blocks, int64_t N, int64_t K, void* out, int out_dtype, void* stream) {
  g_last_error.clear();
  const char* fn = "w4_q4_0_dequantize";
  if (w4_status st = check_q4_0(N, K, blocks, out, fn)) return st;
  if (out_dtype != W4_F32 && out_dtype != W4_BF16) return fail(W4_ERR_INVALID_ARG, "%s: out_dtype must be W4_F32 or W4_BF16", fn);
  return hip_status(w4::launch_q4_0_dequantize(blocks, N, K, out, out_dtype == W4_BF16, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
