// Benchmark support: a plain streaming read, the bandwidth ceiling for the
// decode kernel's loads (the same non-temporal 16-byte load form, no
// arithmetic beyond an xor that keeps the loads live). Not part of the
// attention path.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kThreads = 512;
constexpr int kUnroll = 8;               // 16-byte loads in flight per thread
constexpr int64_t kChunk = 128 * 1024;   // bytes per workgroup, read front to back

// Workgroup b reads bytes [b * kChunk, (b + 1) * kChunk): consecutive lanes
// read consecutive 16-byte words, kUnroll loads in flight per thread.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* __restrict__ buf,
                                                               int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const int64_t begin = static_cast<int64_t>(blockIdx.x) * (kChunk / 16);
  const int64_t end = min(n16, begin + kChunk / 16);
  uint32_t acc = 0;
  for (int64_t i = begin + threadIdx.x; i < end; i += kThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + u * kThreads;
      v[u] = j < end ? load16_stream(buf + 16 * j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) atomicXor(sink, acc);  // practically never taken; keeps the loads
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t blocks = (bytes + kChunk - 1) / kChunk;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  return launch_timed(stream_read_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads),
                      stream, static_cast<const char*>(buf), n16, sink);
}

}  // namespace pa
