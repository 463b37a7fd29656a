// Host-side launchers of the library's kernels (internal interface between
// the C ABI layer and the kernel translation units).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Timing events for the attention kernels' launches on the calling thread
// (both null: plain launches). Set through pa_set_launch_events.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
LaunchEvents& launch_events();

// Launch `kernel`; with launch events set, through hipExtLaunchKernelGGL so
// the events take the kernel's own start and end time stamps.
// lds_bytes of dynamic shared memory per workgroup.
template <typename K, typename... Args>
inline hipError_t launch_timed_lds(K kernel, dim3 grid, dim3 block, size_t lds_bytes,
                                   hipStream_t stream, Args... args) {
  const LaunchEvents& ev = launch_events();
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, args...);
  return hipGetLastError();
}

template <typename K, typename... Args>
inline hipError_t launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t stream, Args... args) {
  return launch_timed_lds(kernel, grid, block, 0, stream, args...);
}

// Everything one decode launch needs, passed to the kernels by value.
struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* ws_ml;   // [S, H, max_parts, 2]: running max (log2 units) and sum per partition
  float* ws_acc;  // [S, H, max_parts, D]: unnormalised output per partition
  int64_t num_blocks;
  float scale_log2;  // scale * log2(e): scores are kept in base-2 exponent units
  int32_t num_seqs;
  int32_t block_size;
  int32_t num_heads;
  int32_t max_blocks;
  int32_t max_ctx;
  int32_t part_tokens;
  int32_t max_parts;
  int32_t out_f32;  // 1: out is fp32; 0: out has the cache dtype
  int32_t stream_loads;  // 1: non-temporal K/V loads; 0: ordinary cached loads
  int32_t waves;  // wavefronts per workgroup of the partition pass (set by its launch)
  const int32_t* seq_order;  // dispatch order of the launch's units (sequences or groups), or null
};

// Groups of consecutive sequences whose block tables agree on a leading
// run of tokens (forks of one prompt): group g is sequences
// group_start[g] .. group_start[g + 1] - 1 (at most kMaxGroup of them), and
// their tables agree on the first group_shared[g] tokens.
constexpr int kMaxGroup = 4;
struct GroupArgs {
  const int32_t* group_start;   // [num_groups + 1]
  const int32_t* group_shared;  // [num_groups], tokens
  int32_t num_groups;
};

enum class Dtype : int { F32 = 0, F16 = 1, BF16 = 2 };

// Tokens one wavefront processes per loop iteration for (dtype, head_dim,
// heads); partition sizes are multiples of it. 0 if the combination is
// unsupported.
int chunk_tokens(Dtype dt, int head_dim, int num_heads);

// Heads per workgroup of the default launch form for (dtype, head_dim,
// heads); 0 if the combination is unsupported.
int heads_per_workgroup(Dtype dt, int head_dim, int num_heads);

// Queue the partition pass / the merge pass. Return a hipError_t.
hipError_t launch_decode_partitions(const DecodeArgs& a, Dtype dt, int head_dim,
                                    hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, Dtype dt, int head_dim, hipStream_t stream);
// The partition pass over groups of sequences (g != nullptr), or the
// ungrouped pass (g == nullptr).
hipError_t launch_decode_groups(const DecodeArgs& a, const GroupArgs* g, Dtype dt, int head_dim,
                                hipStream_t stream);

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int64_t* slots,
                            void* k_cache, void* v_cache, int64_t num_tokens, int64_t row_bytes,
                            int64_t num_slots, hipStream_t stream);

hipError_t launch_kv_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs,
                                 int64_t num_pairs, int64_t frame_bytes, int64_t num_blocks,
                                 hipStream_t stream);

hipError_t launch_gather(const void* cache, const int32_t* block_tables,
                         const int32_t* context_lens, const int64_t* out_row_start, void* out,
                         int32_t num_seqs, int64_t row_bytes, int32_t block_size,
                         int64_t num_blocks, int32_t max_blocks, int32_t max_ctx,
                         hipStream_t stream);

// Streaming-read bandwidth probe (benchmark support).
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace pa
