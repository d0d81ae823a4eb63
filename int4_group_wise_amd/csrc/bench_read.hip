// Streaming-read floor for the decode benchmark (measurement only; not part of
// the w4 library): one launch reads a buffer once with 16-byte non-temporal
// loads, U of them per thread issued together, in the most regular pattern
// there is (a workgroup reads U x 4 KB contiguously).  Its time for the decode
// GEMV's byte count is the rate a single launch of that size reaches on this
// GPU, beside the 8 TB/s peak.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, uint32_t* __restrict__ out) {
  const size_t base = static_cast<size_t>(blockIdx.x) * (256 * U) + threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + base + 256 * u);
  u32x4 acc = v[0];
#pragma unroll
  for (int u = 1; u < U; ++u) acc ^= v[u];
  const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  // the loads feed a store that is almost never taken, so they stay and the
  // kernel writes (next to) nothing
  if (r == 0x9E3779B9u) out[blockIdx.x] = r;
}

template <int U>
hipError_t launch(const void* p, size_t bytes, void* out, hipStream_t s) {
  const size_t per_wg = size_t(256) * U * 16;
  if (bytes % per_wg != 0 || bytes / per_wg > 0x7FFFFFFFu) return hipErrorInvalidValue;
  stream_read_kernel<U><<<dim3(static_cast<uint32_t>(bytes / per_wg)), dim3(256), 0, s>>>(
      static_cast<const u32x4*>(p), static_cast<uint32_t*>(out));
  return hipGetLastError();
}

}  // namespace

// Reads `bytes` bytes at p (16-byte aligned, a multiple of 4096 * unroll) with
// `unroll` (2, 4, 8 or 16) loads per thread; `out` must hold one uint32 per
// workgroup (bytes / (4096 * unroll)).  Returns the HIP error code (0 on
// success; hipErrorInvalidValue for an unsupported size or unroll).
extern "C" int w4bench_stream_read(const void* p, size_t bytes, int unroll, void* out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (unroll) {
    case 2: return launch<2>(p, bytes, out, s);
    case 4: return launch<4>(p, bytes, out, s);
    case 8: return launch<8>(p, bytes, out, s);
    case 16: return launch<16>(p, bytes, out, s);
    default: return hipErrorInvalidValue;
  }
}
