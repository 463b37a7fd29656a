// Host-side launcher of the prefill kernel (internal interface between the C
// ABI layer and paged_prefill.hip).
#pragma once

#include "pa_launch.h"

namespace pa {

// Arguments of the causal multi-query (prefill) kernel.
struct PrefillArgs {
  const void* q;               // [total_queries, H, D]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;  // [S + 1]
  void* out;                   // [total_queries, H, D]
  int64_t num_blocks;
  float scale_log2;            // |scale| * log2(e), >= 0
  int32_t negate_q;            // 1 when scale < 0: q enters with its sign flipped
  int32_t num_seqs;
  int32_t block_size;
  int32_t num_heads;
  int32_t max_blocks;
  int32_t max_ctx;
  int32_t max_query_len;
  int32_t total_queries;
  int32_t out_f32;
  // bf16 caches: 1 = the weights enter the weighted sum as a bf16 value plus
  // its bf16 residual; 0 = V is staged in fp16 and the weights are rounded
  // once to fp16 (a workgroup that meets a V value of magnitude 2^16 or more
  // redoes its work the first way). Unused for fp16 caches.
  int32_t split_weights;
  const int32_t* work_order;   // [S * query tiles] dispatch order of the work items, or null
};

// Queries per prefill work item (the prefill kernel's query tile).
constexpr int kPrefillTile = 128;

bool prefill_supported(Dtype dt, int head_dim);
hipError_t launch_prefill(const PrefillArgs& a, Dtype dt, int head_dim, hipStream_t stream);

}  // namespace pa
