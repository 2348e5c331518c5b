// Streaming-read probe: the practical HBM read rate of the load shape the streaming FFN kernels
// use for their weights -- 16-byte nontemporal loads, consecutive lanes on consecutive 16-byte
// pieces, so that every load instruction of a wave reads 1 KB of whole 128-byte lines.  Reading a
// buffer much larger than the caches with it gives the rate the kernels' weight streams are
// compared with, next to the nominal 8 TB/s.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {
// Each workgroup reads one contiguous 64 KB chunk, eight loads in flight per lane (32 KB per pass of
// the workgroup).  Measured over 4 GiB this shape reads at 7.1-7.2 TB/s; a grid-stride loop over
// 4096 workgroups with four loads in flight reached only 6.6, and ordinary (cached) loads of the
// chunked shape 6.4.
constexpr int kStreamU = 8;
constexpr uint64_t kStreamChunk16 = (64u << 10) / 16;  // pieces per workgroup
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf, uint64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const uint64_t lo = (uint64_t)blockIdx.x * kStreamChunk16;
  const uint64_t hi = lo + kStreamChunk16 < n16 ? lo + kStreamChunk16 : n16;
  uint32_t acc = 0;
  for (uint64_t base = lo + threadIdx.x; base < hi; base += 256u * kStreamU) {
    u32x4 v[kStreamU];
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const uint64_t i = base + 256u * u;
      v[u] = i < hi ? __builtin_nontemporal_load(buf + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) acc ^= v[u][0] + v[u][1] + v[u][2] + v[u][3];
  }
  if (acc == 0x9E3779B9u) *sink = acc;  // (practically never: keeps the loads without a store per thread)
}
}  // namespace

hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t stream) {
  const uint64_t n16 = bytes / 16;
  const uint64_t grid = (n16 + kStreamChunk16 - 1) / kStreamChunk16;
  if (grid > 0x7FFFFFFFu) return hipErrorInvalidValue;  // beyond 128 TiB
  stream_read_kernel<<<(unsigned)grid, 256, 0, stream>>>((const u32x4*)buf, n16, sink);
  return hipGetLastError();
}

}  // namespace moe
