// Streaming-read ceiling of the device: one plain read kernel over a caller's buffer,
// the reference the measured decode rates are also compared with (next to the HBM
// datasheet peak).
#include <string>

#include "ap_internal.h"

namespace ap {

// The loaded words feed one store, taken only when a thread's XOR of them equals a fixed
// constant (then every such thread stores that same constant here), so that the loads
// stay in the program.
__device__ uint32_t g_read_sink;

// Each workgroup reads one contiguous chunk of `per` 16-byte words, 16 loads per thread
// in flight (of the patterns measured on MI355X over 1 GiB, chunks of 64 KB to 1 MB per
// workgroup read fastest, 6.2-6.3 TB/s, against 5.3-5.8 TB/s for a grid-stride loop).
constexpr int kReadThreads = 256, kReadUnroll = 16;
constexpr size_t kReadChunk16 = 16384;   // 256 KB per workgroup

__global__ __launch_bounds__(kReadThreads) void k_read_stream(const uint4* __restrict__ src, size_t n16) {
  const size_t b0 = (size_t)blockIdx.x * kReadChunk16;
  const size_t b1 = b0 + kReadChunk16 < n16 ? b0 + kReadChunk16 : n16;
  uint32_t acc = 0;
  for (size_t i = b0 + threadIdx.x; i < b1; i += (size_t)kReadUnroll * kReadThreads) {
    uint4 x[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const size_t j = i + (size_t)u * kReadThreads;
      x[u] = src[j < b1 ? j : b1 - 1];   // clamped: in bounds, the loads stay unconditional
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  if (acc == 0x9E3779B9u) g_read_sink = acc;
}

}  // namespace ap

using namespace ap;

extern "C" ap_status ap_read_bandwidth(const void* buf, size_t bytes, int32_t passes, void* stream,
                                       float* ms_per_pass) {
  if (!buf || !ms_per_pass) {
    set_error("ap_read_bandwidth: buf and ms_per_pass must not be NULL");
    return AP_ERR_NULL_ARG;
  }
  if (bytes < 16 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0 || passes < 1 ||
      passes > 1000) {
    set_error("ap_read_bandwidth: need a 16-byte aligned buffer of a multiple of 16 bytes, 1 <= passes <= 1000");
    return AP_ERR_BAD_SHAPE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t n16 = bytes / 16;
  const unsigned grid = static_cast<unsigned>((n16 + kReadChunk16 - 1) / kReadChunk16);
  hipError_t e = hipSuccess;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  // one untimed pass, then the timed ones
  if (e == hipSuccess) {
    hipLaunchKernelGGL(k_read_stream, dim3(grid), dim3(kReadThreads), 0, st, static_cast<const uint4*>(buf), n16);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e0, st);
  for (int p = 0; p < passes && e == hipSuccess; ++p) {
    hipLaunchKernelGGL(k_read_stream, dim3(grid), dim3(kReadThreads), 0, st, static_cast<const uint4*>(buf), n16);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, st);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) {
    set_error(std::string("ap_read_bandwidth: ") + hipGetErrorString(e));
    return AP_ERR_HIP;
  }
  *ms_per_pass = ms / static_cast<float>(passes);
  return AP_OK;
}
