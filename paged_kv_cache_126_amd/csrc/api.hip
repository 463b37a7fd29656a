// C ABI of the library (declared in include/paged_attn.h): argument checks,
// launch sizing and dispatch. Every check uses host-known arguments only and
// happens before anything is queued; nothing here synchronises the device.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "paged_attn.h"
#include "pa_launch.h"
#include "pa_prefill.h"
#include "pa_probes.h"

namespace pa {

LaunchEvents& launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}

}  // namespace pa

namespace {

// Default partition size: the largest of 2048, 1024, 512 tokens that still
// yields about kTargetWorkgroups workgroups (32 per compute unit of a 256-CU
// MI355X), estimated from the host-known bound max_context_len. Long
// partitions write fewer partial results; enough workgroups keep every CU
// busy until the end of the launch.
constexpr int32_t kMaxDefaultPartition = 2048;
constexpr int32_t kMinDefaultPartition = 512;
constexpr int64_t kTargetWorkgroups = 8192;
// With a dispatch order (longest work first) the tail is balanced by the
// order, and four workgroups per compute unit suffice.
constexpr int64_t kTargetWorkgroupsOrdered = 1024;
// With a dispatch order, contexts of up to kMaxSinglePartition tokens take
// one partition each when the launch keeps kTargetWorkgroupsOrdered
// workgroups at twice the heads per workgroup (the wide launch form): two
// partitions, the second of them short, ran slower than one (256 sequences
// of up to 4096 bf16 tokens: 1348 us at 2048-token partitions, 1313 us at
// one partition in the wide form).
constexpr int64_t kMaxSinglePartition = 4096;
constexpr int64_t kMaxGridYZ = 65535;
constexpr size_t kWorkspaceAlign = 256;
static_assert(pa::kMaxGroup == PA_MAX_GROUP, "group size limit of the kernels and the header");
static_assert(pa::kPrefillTile == PA_PREFILL_TILE, "prefill work items are query tiles");

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_dtype(pa_dtype d) { return d == PA_F32 || d == PA_F16 || d == PA_BF16; }

int64_t elem_bytes(pa_dtype d) { return d == PA_F32 ? 4 : 2; }

pa::Dtype to_internal(pa_dtype d) {
  return d == PA_F32 ? pa::Dtype::F32 : (d == PA_F16 ? pa::Dtype::F16 : pa::Dtype::BF16);
}

bool supported_head_dim(int32_t d) {
  return d == 16 || d == 32 || d == 64 || d == 128 || d == 256;
}

// Shape validity apart from pointers; fills the partition size and count.
pa_status check_shape(const pa_decode_shape* sh, int32_t* part_tokens, int32_t* max_parts) {
  if (!sh) return PA_EINVAL;
  if (sh->num_seqs < 0 || sh->num_heads <= 0 || sh->block_size <= 0 || sh->num_blocks <= 0 ||
      sh->num_blocks > 0x7FFFFFFFLL ||
      sh->max_blocks_per_seq <= 0 || sh->max_context_len < 0 || sh->partition_tokens < 0)
    return PA_EINVAL;
  if (!supported_head_dim(sh->head_dim) || !valid_dtype(sh->kv_dtype)) return PA_EINVAL;
  if (sh->out_dtype != PA_F32 && sh->out_dtype != sh->kv_dtype) return PA_EINVAL;
  if (static_cast<int64_t>(sh->max_context_len) >
      static_cast<int64_t>(sh->max_blocks_per_seq) * sh->block_size)
    return PA_EINVAL;
  if (sh->num_seqs > kMaxGridYZ) return PA_EINVAL;
  // One frame's bytes must fit 31 bits (the kernels address inside a frame
  // with 32-bit offsets).
  if (static_cast<int64_t>(sh->block_size) * sh->num_heads * sh->head_dim * elem_bytes(sh->kv_dtype) >
      0x7FFFFFFFLL)
    return PA_EINVAL;
  const int chunk = pa::chunk_tokens(to_internal(sh->kv_dtype), sh->head_dim, sh->num_heads);
  if (chunk <= 0) return PA_EINVAL;
  if (sh->cache_policy != PA_CACHE_STREAM && sh->cache_policy != PA_CACHE_REUSE) return PA_EINVAL;
  int64_t pt = sh->partition_tokens;
  if (pt == 0) {
    pt = kMaxDefaultPartition;
    const int64_t pairs = static_cast<int64_t>(sh->num_seqs) * sh->num_heads;
    const int64_t target = sh->dispatch_order ? kTargetWorkgroupsOrdered : kTargetWorkgroups;
    const int hp = pa::heads_per_workgroup(to_internal(sh->kv_dtype), sh->head_dim, sh->num_heads);
    if (sh->dispatch_order && sh->max_context_len > kMaxDefaultPartition &&
        sh->max_context_len <= kMaxSinglePartition && hp > 0 &&
        pairs / (2 * hp) >= kTargetWorkgroupsOrdered) {
      pt = kMaxSinglePartition;  // one partition for every sequence
    } else {
      while (pt > kMinDefaultPartition && pairs * ((sh->max_context_len + pt - 1) / pt) < target)
        pt /= 2;
    }
  }
  pt = (pt + chunk - 1) / chunk * chunk;
  if (pt > (1 << 30)) return PA_EINVAL;
  // partition starts (part * pt) and ends stay in int32
  if (static_cast<int64_t>(sh->max_context_len) + pt > 0x7FFFFFFFLL) return PA_EINVAL;
  int64_t parts = sh->max_context_len <= pt ? 1 : (sh->max_context_len + pt - 1) / pt;
  if (parts > kMaxGridYZ) return PA_EINVAL;
  // The partial results, S * H * parts * (D + 2) floats, must be addressable
  // (this also keeps the workspace size from overflowing size_t).
  const unsigned __int128 partials = static_cast<unsigned __int128>(sh->num_seqs) * sh->num_heads *
                                     static_cast<uint64_t>(parts) * (sh->head_dim + 2) * sizeof(float);
  if (partials > (static_cast<unsigned __int128>(1) << 62)) return PA_EINVAL;
  *part_tokens = static_cast<int32_t>(pt);
  *max_parts = static_cast<int32_t>(parts);
  return PA_OK;
}

size_t ml_bytes(const pa_decode_shape* sh, int32_t max_parts) {
  size_t b = static_cast<size_t>(sh->num_seqs) * sh->num_heads * max_parts * 2 * sizeof(float);
  return (b + kWorkspaceAlign - 1) / kWorkspaceAlign * kWorkspaceAlign;
}

size_t workspace_bytes_for(const pa_decode_shape* sh, int32_t max_parts) {
  if (max_parts <= 1) return 0;
  return ml_bytes(sh, max_parts) +
         static_cast<size_t>(sh->num_seqs) * sh->num_heads * max_parts * sh->head_dim * sizeof(float);
}

pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_EHIP; }

// Points the partial-result arrays of `a` into `workspace` (a buffer of at
// least workspace_bytes_for(sh, a->max_parts) bytes), or at nothing when no
// sequence is split.
void set_workspace(const pa_decode_shape* sh, void* workspace, pa::DecodeArgs* a) {
  const bool split = workspace_bytes_for(sh, a->max_parts) > 0;
  a->ws_ml = split ? static_cast<float*>(workspace) : nullptr;
  a->ws_acc = split ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                               ml_bytes(sh, a->max_parts))
                    : nullptr;
}

// Shared validation and argument packing of the decode entry points. With
// check_workspace false the workspace arguments are ignored and the
// partial-result pointers are left for the caller to set.
pa_status prepare_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         int32_t block_size, float scale, void* out, const pa_decode_shape* sh,
                         void* workspace, size_t workspace_bytes, pa::DecodeArgs* a,
                         bool check_workspace = true) {
  int32_t pt = 0, parts = 0;
  pa_status st = check_shape(sh, &pt, &parts);
  if (st != PA_OK) return st;
  if (block_size != sh->block_size || !std::isfinite(scale)) return PA_EINVAL;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PA_EINVAL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, static_cast<uintptr_t>(elem_bytes(sh->out_dtype))) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(sh->dispatch_order, 4))
    return PA_EALIGN;
  const size_t need = workspace_bytes_for(sh, parts);
  if (check_workspace && need > 0 &&
      (!workspace || workspace_bytes < need || !aligned(workspace, kWorkspaceAlign)))
    return PA_EWORKSPACE;
  a->q = q;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->out = out;
  a->num_blocks = sh->num_blocks;
  a->scale_log2 = scale * 1.4426950408889634f;  // log2(e)
  a->num_seqs = sh->num_seqs;
  a->block_size = sh->block_size;
  a->num_heads = sh->num_heads;
  a->max_blocks = sh->max_blocks_per_seq;
  a->max_ctx = sh->max_context_len;
  a->part_tokens = pt;
  a->max_parts = parts;
  a->out_f32 = sh->out_dtype == PA_F32 ? 1 : 0;
  a->stream_loads = sh->cache_policy == PA_CACHE_STREAM ? 1 : 0;
  a->seq_order = sh->dispatch_order;
  set_workspace(sh, check_workspace ? workspace : nullptr, a);
  return PA_OK;
}

// Scratch of paged_attn_decode_noalloc: the partition partials of one call,
// in a fixed device array instead of a caller's workspace. Each GPU the
// library runs on holds its own copy of the array, at its own address, until
// the process ends. In host code `scratch` names a host-side stand-in, not
// device memory: host code uses only the device address obtained below.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the calling thread's current device, looked
// up once per device (with that device current) and kept.
pa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PA_EHIP;
    if (!aligned(p, kWorkspaceAlign)) return PA_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_EINVAL: return "PA_EINVAL: invalid argument or unsupported shape/dtype";
    case PA_EALIGN: return "PA_EALIGN: misaligned pointer";
    case PA_EWORKSPACE:
      return "PA_EWORKSPACE: workspace missing or too small (paged_attn_decode_noalloc: the "
             "shape needs more than PA_NOALLOC_SCRATCH_BYTES of partial results)";
    case PA_EHIP: return "PA_EHIP: HIP launch error";
  }
  return "unknown pa_status";
}

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

pa_status kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                    void* k_cache, void* v_cache, int64_t num_tokens, int32_t num_heads,
                    int32_t head_dim, int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                    void* stream) {
  if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      num_blocks > 0x7FFFFFFFLL || !valid_dtype(dtype))
    return PA_EINVAL;
  const int64_t row_bytes = static_cast<int64_t>(num_heads) * head_dim * elem_bytes(dtype);
  if ((static_cast<int64_t>(head_dim) * elem_bytes(dtype)) % 16 != 0) return PA_EINVAL;
  if (num_tokens > 0x7FFFFFFF) return PA_EINVAL;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PA_EINVAL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
    return PA_EALIGN;
  return from_hip(pa::launch_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, num_tokens,
                                       row_bytes, num_blocks * block_size,
                                       static_cast<hipStream_t>(stream)));
}

pa_status kv_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs,
                         int64_t num_pairs, int32_t num_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, pa_dtype dtype, void* stream) {
  if (num_pairs < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      num_blocks > 0x7FFFFFFFLL || !valid_dtype(dtype))
    return PA_EINVAL;
  if ((static_cast<int64_t>(head_dim) * elem_bytes(dtype)) % 16 != 0) return PA_EINVAL;
  if (num_pairs > 0x7FFFFFFF) return PA_EINVAL;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) return PA_EINVAL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_pairs, 8)) return PA_EALIGN;
  const int64_t frame_bytes =
      static_cast<int64_t>(block_size) * num_heads * head_dim * elem_bytes(dtype);
  return from_hip(pa::launch_kv_copy_blocks(k_cache, v_cache, block_pairs, num_pairs, frame_bytes,
                                            num_blocks, static_cast<hipStream_t>(stream)));
}

size_t paged_attn_workspace_size(const pa_decode_shape* shape) {
  int32_t pt = 0, parts = 0;
  if (check_shape(shape, &pt, &parts) != PA_OK) return 0;
  return workspace_bytes_for(shape, parts);
}

int32_t paged_attn_partition_tokens(const pa_decode_shape* shape) {
  int32_t pt = 0, parts = 0;
  if (check_shape(shape, &pt, &parts) != PA_OK) return 0;
  return pt;
}

pa_status paged_attn_decode_partitions(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       int32_t block_size, float scale, void* out,
                                       const pa_decode_shape* shape, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  pa::DecodeArgs a;
  pa_status st = prepare_decode(q, k_cache, v_cache, block_tables, context_lens, block_size,
                                scale, out, shape, workspace, workspace_bytes, &a);
  if (st != PA_OK) return st;
  if (shape->num_seqs == 0) return PA_OK;
  return from_hip(pa::launch_decode_partitions(a, to_internal(shape->kv_dtype), shape->head_dim,
                                               static_cast<hipStream_t>(stream)));
}

pa_status paged_attn_merge(const int32_t* context_lens, void* out, const pa_decode_shape* shape,
                           const void* workspace, size_t workspace_bytes, void* stream) {
  int32_t pt = 0, parts = 0;
  pa_status st = check_shape(shape, &pt, &parts);
  if (st != PA_OK) return st;
  if (!context_lens || !out) return PA_EINVAL;
  if (!aligned(out, static_cast<uintptr_t>(elem_bytes(shape->out_dtype))) ||
      !aligned(context_lens, 4))
    return PA_EALIGN;
  const size_t need = workspace_bytes_for(shape, parts);
  if (need == 0 || shape->num_seqs == 0) return PA_OK;  // nothing was split
  if (!workspace || workspace_bytes < need || !aligned(workspace, kWorkspaceAlign))
    return PA_EWORKSPACE;
  pa::DecodeArgs a = {};
  a.context_lens = context_lens;
  a.out = out;
  a.ws_ml = static_cast<float*>(const_cast<void*>(workspace));
  a.ws_acc = reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(workspace)) +
                                      ml_bytes(shape, parts));
  a.num_seqs = shape->num_seqs;
  a.num_heads = shape->num_heads;
  a.max_ctx = shape->max_context_len;
  a.part_tokens = pt;
  a.max_parts = parts;
  a.out_f32 = shape->out_dtype == PA_F32 ? 1 : 0;
  return from_hip(pa::launch_decode_merge(a, to_internal(shape->kv_dtype), shape->head_dim,
                                          static_cast<hipStream_t>(stream)));
}

pa_status paged_attn_decode_grouped(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    int32_t block_size, float scale, void* out,
                                    const pa_decode_shape* shape, const int32_t* group_start,
                                    const int32_t* group_shared, int32_t num_groups,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (num_groups < 0 || num_groups > kMaxGridYZ) return PA_EINVAL;
  pa::DecodeArgs a;
  pa_status st = prepare_decode(q, k_cache, v_cache, block_tables, context_lens, block_size,
                                scale, out, shape, workspace, workspace_bytes, &a);
  if (st != PA_OK) return st;
  if (shape->num_seqs == 0 || num_groups == 0) return PA_OK;
  if (!group_start || !group_shared) return PA_EINVAL;
  if (!aligned(group_start, 4) || !aligned(group_shared, 4)) return PA_EALIGN;
  pa::GroupArgs g;
  g.group_start = group_start;
  g.group_shared = group_shared;
  g.num_groups = num_groups;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = from_hip(pa::launch_decode_groups(a, &g, to_internal(shape->kv_dtype), shape->head_dim, s));
  if (st != PA_OK) return st;
  return paged_attn_merge(context_lens, out, shape, workspace, workspace_bytes, stream);
}

pa_status paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t block_size, float scale, void* out,
                            const pa_decode_shape* shape, void* workspace,
                            size_t workspace_bytes, void* stream) {
  pa_status st = paged_attn_decode_partitions(q, k_cache, v_cache, block_tables, context_lens,
                                              block_size, scale, out, shape, workspace,
                                              workspace_bytes, stream);
  if (st != PA_OK) return st;
  return paged_attn_merge(context_lens, out, shape, workspace, workspace_bytes, stream);
}

pa_status paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    int32_t block_size, float scale, void* out,
                                    const pa_decode_shape* shape, void* stream) {
  pa::DecodeArgs a;
  pa_status st = prepare_decode(q, k_cache, v_cache, block_tables, context_lens, block_size,
                                scale, out, shape, nullptr, 0, &a, /*check_workspace=*/false);
  if (st != PA_OK) return st;
  const size_t need = workspace_bytes_for(shape, a.max_parts);
  if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_EWORKSPACE;
  if (shape->num_seqs == 0) return PA_OK;
  if (need > 0) {
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != PA_OK) return st;
    set_workspace(shape, ws, &a);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const pa::Dtype dt = to_internal(shape->kv_dtype);
  st = from_hip(pa::launch_decode_partitions(a, dt, shape->head_dim, s));
  if (st != PA_OK || need == 0) return st;
  return from_hip(pa::launch_decode_merge(a, dt, shape->head_dim, s));
}

pa_status paged_attn_prefill(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             const int32_t* query_start, int32_t block_size, float scale,
                             void* out, const pa_prefill_shape* sh, const int32_t* work_order,
                             void* stream) {
  if (!sh) return PA_EINVAL;
  if (sh->num_seqs < 0 || sh->num_heads <= 0 || sh->block_size <= 0 || sh->num_blocks <= 0 ||
      sh->num_blocks > 0x7FFFFFFFLL || sh->max_blocks_per_seq <= 0 || sh->max_context_len < 0 ||
      sh->max_query_len < 0 || sh->total_queries < 0 || !valid_dtype(sh->kv_dtype))
    return PA_EINVAL;
  if (!pa::prefill_supported(to_internal(sh->kv_dtype), sh->head_dim)) return PA_EINVAL;
  if (sh->out_dtype != PA_F32 && sh->out_dtype != sh->kv_dtype) return PA_EINVAL;
  if (block_size != sh->block_size || !std::isfinite(scale)) return PA_EINVAL;
  if (sh->split_weights != 0 && sh->split_weights != 1) return PA_EINVAL;
  if (static_cast<int64_t>(sh->max_context_len) >
      static_cast<int64_t>(sh->max_blocks_per_seq) * sh->block_size)
    return PA_EINVAL;
  if (static_cast<int64_t>(sh->block_size) * sh->num_heads * sh->head_dim * elem_bytes(sh->kv_dtype) >
      0x7FFFFFFFLL)
    return PA_EINVAL;
  const int64_t query_tiles = (static_cast<int64_t>(sh->max_query_len) + PA_PREFILL_TILE - 1) /
                              PA_PREFILL_TILE;
  if (sh->num_seqs * query_tiles * sh->num_heads > 0x7FFFFFFFLL) return PA_EINVAL;
  if (sh->num_seqs == 0 || sh->max_query_len == 0 || sh->total_queries == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
    return PA_EINVAL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, static_cast<uintptr_t>(elem_bytes(sh->out_dtype))) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4) ||
      !aligned(work_order, 4))
    return PA_EALIGN;
  pa::PrefillArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.out = out;
  a.num_blocks = sh->num_blocks;
  // The kernel takes each query's maximum on unscaled scores, which needs a
  // scale >= 0; a negative scale is moved into q, whose sign flip is exact.
  a.scale_log2 = std::fabs(scale) * 1.4426950408889634f;
  a.negate_q = scale < 0.f ? 1 : 0;
  a.num_seqs = sh->num_seqs;
  a.block_size = sh->block_size;
  a.num_heads = sh->num_heads;
  a.max_blocks = sh->max_blocks_per_seq;
  a.max_ctx = sh->max_context_len;
  a.max_query_len = sh->max_query_len;
  a.total_queries = sh->total_queries;
  a.out_f32 = sh->out_dtype == PA_F32 ? 1 : 0;
  a.split_weights = sh->split_weights;
  a.work_order = work_order;
  return from_hip(pa::launch_prefill(a, to_internal(sh->kv_dtype), sh->head_dim,
                                     static_cast<hipStream_t>(stream)));
}

pa_status paged_gather(const void* cache, const int32_t* block_tables,
                       const int32_t* context_lens, const int64_t* out_row_start, void* out,
                       int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size,
                       int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                       pa_dtype dtype, void* stream) {
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      num_blocks > 0x7FFFFFFFLL || max_blocks_per_seq <= 0 || max_context_len < 0 || !valid_dtype(dtype))
    return PA_EINVAL;
  if ((static_cast<int64_t>(head_dim) * elem_bytes(dtype)) % 16 != 0) return PA_EINVAL;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PA_EINVAL;
  if (num_seqs > kMaxGridYZ) return PA_EINVAL;
  if (num_seqs == 0 || max_context_len == 0) return PA_OK;
  if (!cache || !block_tables || !context_lens || !out_row_start || !out) return PA_EINVAL;
  if (!aligned(cache, 16) || !aligned(out, 16) || !aligned(block_tables, 4) ||
      !aligned(context_lens, 4) || !aligned(out_row_start, 8))
    return PA_EALIGN;
  const int64_t row_bytes = static_cast<int64_t>(num_heads) * head_dim * elem_bytes(dtype);
  return from_hip(pa::launch_gather(cache, block_tables, context_lens, out_row_start, out,
                                    num_seqs, row_bytes, block_size, num_blocks,
                                    max_blocks_per_seq, max_context_len,
                                    static_cast<hipStream_t>(stream)));
}

pa_status pa_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || (bytes > 0 && (!buf || !sink))) return PA_EINVAL;
  if (bytes == 0) return PA_OK;
  if (!aligned(buf, 16)) return PA_EALIGN;
  return from_hip(pa::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

pa_status pa_frame_read(const void* buf, int64_t bytes, const int32_t* frame_order,
                        int64_t num_frames, int64_t frame_bytes, int32_t groups,
                        int64_t group_stride, int32_t pieces, int64_t piece_stride,
                        int32_t piece_bytes, int32_t frames_per_unit, uint32_t* sink,
                        void* stream) {
  if (bytes < 0 || num_frames < 0 || frame_bytes <= 0 || groups <= 0 || pieces <= 0 ||
      piece_bytes <= 0 || frames_per_unit <= 0 || group_stride < 0 || piece_stride < 0)
    return PA_EINVAL;
  if (frame_bytes % 16 || group_stride % 16 || piece_stride % 16 || piece_bytes % 16)
    return PA_EINVAL;
  if (frame_bytes > (int64_t{1} << 40) || group_stride > frame_bytes || piece_stride > frame_bytes)
    return PA_EINVAL;
  // every piece lies inside its frame, every frame inside the buffer
  if (static_cast<int64_t>(groups - 1) * group_stride + static_cast<int64_t>(pieces - 1) * piece_stride +
          piece_bytes > frame_bytes)
    return PA_EINVAL;
  if (num_frames > bytes / frame_bytes) return PA_EINVAL;
  if (static_cast<int64_t>(pieces) * (piece_bytes / 16) > 0x7FFFFFFFLL) return PA_EINVAL;
  if ((num_frames + frames_per_unit - 1) / frames_per_unit > kMaxGridYZ) return PA_EINVAL;
  if (num_frames == 0) return PA_OK;
  if (!buf || !frame_order || !sink) return PA_EINVAL;
  if (!aligned(buf, 16) || !aligned(frame_order, 4) || !aligned(sink, 4)) return PA_EALIGN;
  return from_hip(pa::launch_frame_read(buf, frame_order, num_frames, frame_bytes, groups,
                                        group_stride, pieces, piece_stride, piece_bytes,
                                        frames_per_unit, sink, static_cast<hipStream_t>(stream)));
}

pa_status pa_set_launch_events(void* start, void* stop) {
  pa::launch_events() = {static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)};
  return PA_OK;
}

}  // extern "C"
