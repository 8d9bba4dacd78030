// Streaming-read probe: the device's practical read bandwidth, the ceiling
// next to which the bandwidth-bound decode kernels are measured (the spec
// peak is never reached by a real read stream).  Every 16-byte word of the source is loaded
// exactly once, eight independent loads in flight per thread.  The loads are
// non-temporal: for a pure contiguous stream they run about 10% faster than
// plain loads (6.6-6.9 against 6.0-6.3 TB/s over 512 MiB), so the probe gives
// the best read rate the device reaches, not the rate of the decode's own
// load flavour.
#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

// Each workgroup reads one contiguous run of 256 * kProbeUnroll 16-byte words,
// every load issued before the first use; the grid covers the source once.
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * 256 * kProbeUnroll + threadIdx.x;
  u32x4 w[kProbeUnroll];
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) {
    const int64_t i = base + (int64_t)u * 256;
    w[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
  }
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) acc ^= w[u];
  // Keeps the loads live; the written value carries no meaning.
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9E3779B9u) *sink = x;
}

}  // namespace

int launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t nwg = (n16 + 256 * kProbeUnroll - 1) / (256 * kProbeUnroll);
  if (nwg <= 0) return 0;
  if (nwg > INT32_MAX) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)nwg), dim3(256), 0, stream,
                     (const u32x4*)src, n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace pa
