// Benchmark support: a plain streaming read, the bandwidth ceiling for the
// decode kernel's loads (the same non-temporal 16-byte load form, no
// arithmetic beyond an xor that keeps the loads live), and a frame-pattern
// read that reads a buffer of frames in a given order, one group of pieces
// (one head's rows) at a time, to compare cache layouts on the HBM side.
// Not part of the attention path.
#include "pa_device.h"
#include "pa_launch.h"
#include "pa_probes.h"

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

// Frame-pattern read: workgroup (group g, unit u) reads, for each of the
// unit's frames f = frame_order[u * frames_per_unit + i], the `pieces`
// pieces of piece_bytes at f * frame_bytes + g * group_stride +
// p * piece_stride. Its 8 wavefronts take the unit's frames round robin and
// read each frame's pieces with 16-byte non-temporal loads, 4 in flight per
// lane, as the decode kernel reads one head's rows of a frame.
struct FrameReadArgs {
  const char* buf;
  const int32_t* frame_order;
  int64_t num_frames;
  int64_t frame_bytes;
  int64_t group_stride;
  int64_t piece_stride;
  int32_t pieces;
  int32_t piece_words;  // piece_bytes / 16
  int32_t frames_per_unit;
  uint32_t* sink;
};

constexpr int kFrameWaves = 8;
constexpr int kFrameUnroll = 4;

__global__ __launch_bounds__(kFrameWaves * 64) void frame_read_kernel(FrameReadArgs a) {
  const int g = blockIdx.x;
  const int64_t unit_first = static_cast<int64_t>(blockIdx.y) * a.frames_per_unit;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int words = a.pieces * a.piece_words;  // 16-byte words of one frame's group
  const int64_t n_here = min(static_cast<int64_t>(a.frames_per_unit), a.num_frames - unit_first);
  uint32_t acc = 0;
  for (int64_t i = wave; i < n_here; i += kFrameWaves) {
    int64_t f = a.frame_order[unit_first + i];
    f = f < 0 ? 0 : (f >= a.num_frames ? a.num_frames - 1 : f);  // clamped into the buffer
    const char* base = a.buf + f * a.frame_bytes + static_cast<int64_t>(g) * a.group_stride;
    for (int w0 = lane; w0 < words; w0 += 64 * kFrameUnroll) {
      u32x4 v[kFrameUnroll];
#pragma unroll
      for (int u = 0; u < kFrameUnroll; ++u) {
        const int w = w0 + 64 * u;
        const int p = w / a.piece_words;
        const int o = w - p * a.piece_words;
        v[u] = w < words ? load16_stream(base + p * a.piece_stride + 16 * o) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kFrameUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (acc == 0x9E3779B9u) atomicXor(a.sink, acc);  // practically never taken; keeps the loads
}

}  // namespace

hipError_t launch_frame_read(const void* buf, const int32_t* frame_order, int64_t num_frames,
                             int64_t frame_bytes, int32_t groups, int64_t group_stride,
                             int32_t pieces, int64_t piece_stride, int32_t piece_bytes,
                             int32_t frames_per_unit, uint32_t* sink, hipStream_t stream) {
  FrameReadArgs a;
  a.buf = static_cast<const char*>(buf);
  a.frame_order = frame_order;
  a.num_frames = num_frames;
  a.frame_bytes = frame_bytes;
  a.group_stride = group_stride;
  a.piece_stride = piece_stride;
  a.pieces = pieces;
  a.piece_words = piece_bytes / 16;
  a.frames_per_unit = frames_per_unit;
  a.sink = sink;
  const int64_t units = (num_frames + frames_per_unit - 1) / frames_per_unit;
  if (units > 65535 || groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  return launch_timed(frame_read_kernel, dim3(static_cast<uint32_t>(groups), static_cast<uint32_t>(units)),
                      dim3(kFrameWaves * 64), stream, a);
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t blocks = (bytes + kChunk - 1) / kChunk;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  return launch_timed(stream_read_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads),
                      stream, static_cast<const char*>(buf), n16, sink);
}

}  // namespace pa
