// Block translation as an explicit gather (a checking aid, not the hot path).
//
// For token i of sequence s the source row is frame block_tables[s][i / B] at
// offset i % B ("PagedAttention: Virtual Memory Guide for LLM Inference",
// "The Mathematics of Block Translation"), resolved by the same device
// routine (token_row) as the decode kernel's general path. The copy is
// bit-exact.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void gather_kernel(const char* __restrict__ cache,
                                                     const int32_t* __restrict__ block_tables,
                                                     const int32_t* __restrict__ context_lens,
                                                     const int64_t* __restrict__ out_row_start,
                                                     char* __restrict__ out, int64_t row_bytes,
                                                     int32_t block_size, int64_t num_blocks,
                                                     int32_t max_blocks, int32_t max_ctx) {
  const int32_t i = blockIdx.x;
  const int32_t s = blockIdx.y;
  int32_t ctx = context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > max_ctx ? max_ctx : ctx);
  if (i >= ctx) return;
  const int64_t row = token_row(block_tables + static_cast<int64_t>(s) * max_blocks, i,
                                block_size, num_blocks);
  const int64_t src = row * row_bytes;
  const int64_t dst = (out_row_start[s] + i) * row_bytes;
  for (int64_t c = threadIdx.x; c < row_bytes / 16; c += blockDim.x)
    store16(out + dst + 16 * c, load16(cache + src + 16 * c));
}

}  // namespace

hipError_t launch_gather(const void* cache, const int32_t* block_tables,
                         const int32_t* context_lens, const int64_t* out_row_start, void* out,
                         int32_t num_seqs, int64_t row_bytes, int32_t block_size,
                         int64_t num_blocks, int32_t max_blocks, int32_t max_ctx,
                         hipStream_t stream) {
  const int64_t vecs = row_bytes / 16;
  const int threads = vecs >= 256 ? 256 : static_cast<int>((vecs + 63) / 64 * 64);
  dim3 grid(static_cast<uint32_t>(max_ctx), static_cast<uint32_t>(num_seqs));
  hipLaunchKernelGGL(gather_kernel, grid, dim3(threads), 0, stream,
                     static_cast<const char*>(cache), block_tables, context_lens, out_row_start,
                     static_cast<char*>(out), row_bytes, block_size, num_blocks, max_blocks,
                     max_ctx);
  return hipGetLastError();
}

}  // namespace pa
