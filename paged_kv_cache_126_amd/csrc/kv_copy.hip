// Frame copy for copy-on-write (gfx950).
//
// "PagedAttention: Virtual Memory Guide for LLM Inference", "2. Zero-Copy
// Branching via Copy-on-Write": when a branch must modify a frame that other
// branches still reference, only that one frame is duplicated; every other
// frame stays shared. The host block manager picks the new frame; this kernel
// moves the bytes: frame src of both caches is copied to frame dst.
//
// One workgroup per (pair, slice of the frame); 16-byte vector copies; the
// pair is read as a scalar. A pair with a frame outside [0, num_blocks) is
// skipped.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void kv_copy_blocks_kernel(char* __restrict__ k_cache,
                                                             char* __restrict__ v_cache,
                                                             const int64_t* __restrict__ pairs,
                                                             int64_t frame_bytes,
                                                             int64_t num_blocks) {
  const int64_t n = blockIdx.x;
  const int64_t src = pairs[2 * n];
  const int64_t dst = pairs[2 * n + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t vecs = frame_bytes / 16;
  const int64_t s0 = src * frame_bytes, d0 = dst * frame_bytes;
  for (int64_t c = static_cast<int64_t>(blockIdx.y) * blockDim.x + threadIdx.x; c < vecs;
       c += static_cast<int64_t>(gridDim.y) * blockDim.x) {
    const u32x4 kv = load16(k_cache + s0 + 16 * c);
    const u32x4 vv = load16(v_cache + s0 + 16 * c);
    store16(k_cache + d0 + 16 * c, kv);
    store16(v_cache + d0 + 16 * c, vv);
  }
}

}  // namespace

hipError_t launch_kv_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs,
                                 int64_t num_pairs, int64_t frame_bytes, int64_t num_blocks,
                                 hipStream_t stream) {
  const int64_t vecs = frame_bytes / 16;
  int64_t gy = (vecs + 255) / 256;
  if (gy > 64) gy = 64;  // each thread copies several vectors of a large frame
  dim3 grid(static_cast<uint32_t>(num_pairs), static_cast<uint32_t>(gy));
  hipLaunchKernelGGL(kv_copy_blocks_kernel, grid, dim3(256), 0, stream, static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), pairs, frame_bytes, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
