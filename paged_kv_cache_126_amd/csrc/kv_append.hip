// KV append for gfx950: copy each new token's K and V rows into its slot.
//
// "Solving the LLM Memory Wall: A Deep Dive into PagedAttention",
// "Implementation": writing a token stores its [heads, head_dim] K and V rows
// at [frame, offset] of caches laid out [num_blocks, block_size, heads,
// head_dim]. Since frame * B + offset is the slot, a token's destination row
// is simply row `slot` of the cache viewed as [num_blocks * B, H * D]; the
// write position inside the frame is offset t mod B as "PagedAttention:
// Virtual Memory Guide for LLM Inference" ("1. Demand Paging during
// Autoregressive Decoding") describes.
//
// One workgroup per token (blockIdx.x), threads over the row's 16-byte
// vectors; the slot is a scalar load. The copy is bit-exact: the bytes are
// moved, never converted.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void kv_append_kernel(const char* __restrict__ k_new,
                                                        const char* __restrict__ v_new,
                                                        const int64_t* __restrict__ slots,
                                                        char* __restrict__ k_cache,
                                                        char* __restrict__ v_cache,
                                                        int64_t row_bytes, int64_t num_slots) {
  const int64_t n = blockIdx.x;
  const int64_t slot = slots[n];
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool
  const int64_t vecs = row_bytes / 16;
  const int64_t src = n * row_bytes;
  const int64_t dst = slot * row_bytes;
  for (int64_t c = static_cast<int64_t>(blockIdx.y) * blockDim.x + threadIdx.x; c < vecs;
       c += static_cast<int64_t>(gridDim.y) * blockDim.x) {
    const u32x4 kv = load16(k_new + src + 16 * c);
    const u32x4 vv = load16(v_new + src + 16 * c);
    store16(k_cache + dst + 16 * c, kv);
    store16(v_cache + dst + 16 * c, vv);
  }
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int64_t* slots,
                            void* k_cache, void* v_cache, int64_t num_tokens, int64_t row_bytes,
                            int64_t num_slots, hipStream_t stream) {
  const int64_t vecs = row_bytes / 16;
  const int threads = vecs >= 256 ? 256 : static_cast<int>((vecs + 63) / 64 * 64);
  int64_t gy = (vecs + threads - 1) / threads;
  if (gy > 65535) gy = 65535;
  dim3 grid(static_cast<uint32_t>(num_tokens), static_cast<uint32_t>(gy));
  hipLaunchKernelGGL(kv_append_kernel, grid, dim3(threads), 0, stream,
                     static_cast<const char*>(k_new), static_cast<const char*>(v_new), slots,
                     static_cast<char*>(k_cache), static_cast<char*>(v_cache), row_bytes,
                     num_slots);
  return hipGetLastError();
}

}  // namespace pa
