/*
 * paged_attn.h - C ABI of the paged decode-attention library (AMD gfx950).
 *
 * The library implements the device-side hot path of PagedAttention:
 *
 *   kv_append          writes each new token's K and V rows into the slot the
 *                      host block manager chose for it;
 *   paged_attn_decode  single-query scaled dot-product attention of every
 *                      sequence over its tokens, fetched from fixed-size
 *                      physical frames through a block table.
 *
 * Definitions followed (by page title and section):
 *   - "PagedAttention: Virtual Memory Guide for LLM Inference", section "The
 *     Mathematics of Block Translation": token i of a sequence is in logical
 *     block floor(i / B) at offset i mod B; the block table maps the logical
 *     block to a physical frame. Section "3. PagedAttention CUDA Kernel
 *     Execution": the attention kernel takes the block table directly and
 *     resolves addresses itself, with no gather into a temporary buffer.
 *   - "Solving the LLM Memory Wall: A Deep Dive into PagedAttention", section
 *     "1. The Mathematical Foundation": the result is ordinary softmax
 *     attention, o = sum_j softmax_j(q . k_j * scale) v_j; section
 *     "Implementation": K and V caches are [num_blocks, block_size, heads,
 *     head_dim], and writing a token stores its [heads, head_dim] rows at
 *     [frame, offset].
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers, owned by the caller. The library
 *     allocates nothing, keeps no pointer after returning, and never
 *     synchronises the host: work is queued on `stream` (a hipStream_t; NULL
 *     means the default stream) and results are visible once the stream
 *     reaches that point.
 *   - Tensors are dense and row-major in the shapes given below. Base
 *     pointers of q, k_cache, v_cache, k_new, v_new and out must be 16-byte
 *     aligned; head_dim * element size must be a multiple of 16 bytes.
 *   - Errors are detected on the host from the arguments alone, before any
 *     launch; a call that returns an error has queued nothing.
 *   - Element types: q, k_cache, v_cache, k_new and v_new share one dtype.
 *     Accumulation is fp32.
 *
 * Device-side preconditions (not checked, since checking them would need a
 * device-to-host copy; breaking them yields unspecified results but never an
 * access outside the buffers):
 *   - 0 <= context_lens[s] <= max_context_len; larger values are clamped to
 *     max_context_len and negative values to 0;
 *   - block_tables[s][b] is a frame in [0, num_blocks) for every
 *     b < ceil(context_lens[s] / B); out-of-range entries are clamped into
 *     the pool; entries past that column are never read;
 *   - the slots of one kv_append call are distinct (two tokens written to one
 *     slot race).
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 5

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2
} pa_dtype;

/* How the decode kernel reads the caches. */
typedef enum pa_cache_policy {
  PA_CACHE_STREAM = 0,  /* each frame is read once per call: non-temporal loads
                           that leave the caches to other data (default) */
  PA_CACHE_REUSE = 1    /* sequences of the call share frames (forked prefixes):
                           ordinary loads, so a frame read for one sequence can
                           be served from cache for the others */
} pa_cache_policy;

typedef enum pa_status {
  PA_OK = 0,
  PA_EINVAL = -1,      /* null pointer, non-positive size, or an unsupported
                          dtype / head_dim combination */
  PA_EALIGN = -2,      /* a base pointer is not 16-byte aligned */
  PA_EWORKSPACE = -3,  /* workspace missing, misaligned or too small */
  PA_EHIP = -4         /* the HIP runtime reported an error for the launch */
} pa_status;

/*
 * Size limits, checked on the host (PA_EINVAL beyond them): num_blocks at
 * most 2^31 - 1 in every entry point; one frame, B * H * D * element bytes,
 * under 2^31 bytes (decode and prefill address inside a frame with 32-bit
 * offsets); decode: S and the partition count at most 65,535 each and the
 * partial results, S * H * partitions * (D + 2) * 4 bytes, at most 2^62;
 * prefill: as stated at paged_attn_prefill.
 */

/* Shapes and types of one decode call. */
typedef struct pa_decode_shape {
  int32_t num_seqs;            /* S: queries, one per sequence */
  int32_t num_heads;           /* H: query heads == KV heads */
  int32_t head_dim;            /* D: 16, 32, 64, 128 or 256 */
  int32_t block_size;          /* B: tokens per frame, >= 1 */
  int64_t num_blocks;          /* NB: frames in each cache */
  int32_t max_blocks_per_seq;  /* row stride of block_tables, >= ceil(max_context_len / B) */
  int32_t max_context_len;     /* host-known bound on context_lens; sizes the launch */
  pa_dtype kv_dtype;           /* dtype of q, k_cache and v_cache */
  pa_dtype out_dtype;          /* PA_F32, or kv_dtype (rounded to nearest even) */
  int32_t partition_tokens;    /* tokens per context partition; 0 = chosen by the
                                  library from the shape. Rounded up to what the
                                  kernel's tiling needs. */
  int32_t cache_policy;        /* a pa_cache_policy value */
  const int32_t* dispatch_order; /* NULL, or a device int32 array: the order in
                                  which the launch's units are dispatched, a
                                  permutation of their indices (sequences 0 .. S-1;
                                  groups 0 .. num_groups-1 for
                                  paged_attn_decode_grouped). Values are clamped
                                  into range; a unit missing from it gets no output.
                                  Longest work first shortens the launch's tail;
                                  sequences that share frames (forks of one
                                  prompt) should stay adjacent in it, or their
                                  shared reads drift apart in time and miss in
                                  cache. With an order the default partition
                                  size also grows (see
                                  paged_attn_partition_tokens).
                                  Outputs equal the unordered call's at the same
                                  partition size, bit for bit. */
} pa_decode_shape;

/* Human-readable name of a status code. Never NULL. */
const char* pa_status_string(pa_status status);

/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

/*
 * kv_append: store new tokens' K and V rows in their cache slots.
 *
 *   k_new, v_new   [num_tokens, H, D] in `dtype`
 *   slot_mapping   [num_tokens] int64: slot = frame * B + offset
 *   k_cache,
 *   v_cache        [num_blocks, B, H, D] in `dtype`, updated in place
 *
 * Token n's rows are copied bit for bit to k_cache[slot / B][slot % B] and
 * v_cache[slot / B][slot % B]. A negative slot marks padding and is skipped,
 * as is a slot >= num_blocks * B. num_tokens == 0 queues nothing and
 * returns PA_OK. ("Solving the LLM Memory Wall", "Implementation", the cache
 * update of one token; "PagedAttention: Virtual Memory Guide", "1. Demand
 * Paging during Autoregressive Decoding", the write at offset t mod B.)
 */
pa_status kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                    void* k_cache, void* v_cache, int64_t num_tokens, int32_t num_heads,
                    int32_t head_dim, int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                    void* stream);

/*
 * kv_copy_blocks: copy whole frames, for copy-on-write.
 *
 *   k_cache, v_cache  [num_blocks, B, H, D] in `dtype`, updated in place
 *   block_pairs       [num_pairs, 2] int64 (device): (src frame, dst frame)
 *
 * For each pair, frame src of both caches is copied bit for bit to frame dst
 * (B * H * D elements each). A pair naming a frame outside [0, num_blocks)
 * is skipped. Destination frames must be distinct and must not be the source
 * of another pair in the same call (copies run concurrently).
 * num_pairs == 0 queues nothing. ("PagedAttention: Virtual Memory Guide",
 * "2. Zero-Copy Branching via Copy-on-Write": a branch about to modify a
 * shared frame gets a private copy of that one frame.)
 */
pa_status kv_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs,
                         int64_t num_pairs, int32_t num_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, pa_dtype dtype, void* stream);

/*
 * Workspace bytes paged_attn_decode needs for `shape` (partial results of
 * context partitions); 0 when every sequence fits one partition. Returns 0
 * for an invalid shape too: validate through paged_attn_decode.
 */
size_t paged_attn_workspace_size(const pa_decode_shape* shape);

/*
 * Partition size (tokens) the library uses for `shape`; 0 if invalid. The
 * default is the largest of 2048, 1024 and 512 tokens that still gives about
 * 8,192 workgroups (S * H * partitions of the longest context), or, with a
 * dispatch_order, about 1,024: longest-first dispatch balances long
 * partitions, which write fewer partial results and often need no merge.
 * With a dispatch_order and a max_context_len of 2049-4096 tokens it is
 * 4096 (one partition per sequence) when S * H / (2 * heads per workgroup)
 * is still 1,024 or more.
 */
int32_t paged_attn_partition_tokens(const pa_decode_shape* shape);

/*
 * paged_attn_decode: decode attention through block tables.
 *
 *   q             [S, H, D] in kv_dtype: one query per sequence and head
 *   k_cache,
 *   v_cache       [NB, B, H, D] in kv_dtype
 *   block_tables  [S, max_blocks_per_seq] int32: logical block -> frame
 *   context_lens  [S] int32: tokens each query attends to (its own included)
 *   block_size    B (must equal shape->block_size)
 *   scale         multiplier of q . k (1 / sqrt(D) for standard attention):
 *                 any finite value, zero and negative ones included; a
 *                 non-finite scale is PA_EINVAL
 *   out           [S, H, D] in out_dtype
 *   workspace     device buffer of workspace_bytes >= paged_attn_workspace_size,
 *                 256-byte aligned; may be NULL when that size is 0
 *
 * out[s][h] = sum_{i < ctx} w_i v_i / sum_{i < ctx} w_i with
 * w_i = exp(scale * q[s][h] . k_i - max), k_i and v_i read at frame
 * block_tables[s][i / B], offset i % B, head h. A sequence with ctx == 0
 * gets a zero output. Long contexts are split into partitions processed in
 * parallel and merged by a log-sum-exp reduction (the two kernels run back
 * to back on `stream`).
 */
pa_status paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t block_size, float scale, void* out,
                            const pa_decode_shape* shape, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_noalloc: paged_attn_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments and results as
 * paged_attn_decode (bit for bit, at the same shape), without the
 * workspace: the partition partials go to a fixed scratch array of
 * PA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on,
 * from the first call on that GPU (which looks up the array's device
 * address) until the process ends. The call allocates nothing.
 *
 *   The scratch of the device current on the calling thread is used;
 *   `stream` must belong to that device.
 *   Errors: as paged_attn_decode, plus PA_EWORKSPACE when the shape needs more
 *   partial results than the scratch holds (paged_attn_workspace_size(shape)
 *   > PA_NOALLOC_SCRATCH_BYTES; a larger partition_tokens needs fewer), and
 *   PA_EHIP when the scratch's device address cannot be obtained. Both are
 *   detected before anything is queued.
 *   Every call on one GPU shares that GPU's scratch, which keeps the last
 *   call's contents: calls whose work overlaps in time on one GPU (other
 *   streams, other threads) race and give undefined results; calls queued
 *   in order on one stream are safe. Nothing in the scratch needs clearing:
 *   the partition pass writes every partial the merge pass reads.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
pa_status paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    int32_t block_size, float scale, void* out,
                                    const pa_decode_shape* shape, void* stream);

/*
 * The two launches of paged_attn_decode, exposed separately (same arguments
 * and rules): the partition pass writes `out` for sequences that fit one
 * partition and partial results to `workspace` for the others; the merge
 * pass combines those partials into `out`. Calling both in order on one
 * stream is exactly paged_attn_decode.
 */
pa_status paged_attn_decode_partitions(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       int32_t block_size, float scale, void* out,
                                       const pa_decode_shape* shape, void* workspace,
                                       size_t workspace_bytes, void* stream);

pa_status paged_attn_merge(const int32_t* context_lens, void* out, const pa_decode_shape* shape,
                           const void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped decode: paged_attn_decode for batches in which groups of
 * sequences share the first frames of their block tables (the branches of
 * one prompt after forks: "PagedAttention: Virtual Memory Guide for LLM
 * Inference", "2. Zero-Copy Branching via Copy-on-Write"). One workgroup
 * serves a whole group: each shared K/V row is read from memory once and
 * folded into every member's softmax; the members' own rows are read as
 * usual. Same shape rules, partition size and workspace as
 * paged_attn_decode, and the same outputs, bit for bit.
 *
 *   group_start   device int32 [num_groups + 1]: group g is the batch's
 *                 sequences group_start[g] .. group_start[g + 1] - 1, at most
 *                 4 of them (PA_MAX_GROUP). Groups must cover every
 *                 sequence exactly once: the output of a sequence in no
 *                 group (or past a group's 4th member) is undefined, and
 *                 one in two groups is written twice. Values are clamped
 *                 into [0, S], so no access leaves the buffers.
 *   group_shared  device int32 [num_groups]: tokens the members share. The
 *                 first ceil(group_shared[g] / B) entries of the members'
 *                 block-table rows must be equal; the shared length is cut
 *                 to the shortest member's context. If the rows differ
 *                 there, the shared tokens are read through the first
 *                 member's row (never outside the cache).
 *   num_groups    0 .. 65535
 *
 * The call queues the grouped partition pass and the merge pass on
 * `stream`. Errors: as paged_attn_decode;
 * PA_EINVAL for a negative or too large num_groups or missing group arrays,
 * PA_EALIGN for misaligned ones.
 */
#define PA_MAX_GROUP 4
pa_status paged_attn_decode_grouped(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    int32_t block_size, float scale, void* out,
                                    const pa_decode_shape* shape, const int32_t* group_start,
                                    const int32_t* group_shared, int32_t num_groups,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Shapes and types of one prefill call. */
typedef struct pa_prefill_shape {
  int32_t num_seqs;            /* S */
  int32_t num_heads;           /* H */
  int32_t head_dim;            /* D: 64 or 128 */
  int32_t block_size;          /* B */
  int64_t num_blocks;          /* NB */
  int32_t max_blocks_per_seq;  /* row stride of block_tables */
  int32_t max_context_len;     /* host-known bound on context_lens */
  int32_t max_query_len;       /* host-known bound on queries per sequence; sizes the launch */
  int32_t total_queries;       /* T: rows of q and out */
  pa_dtype kv_dtype;           /* PA_F16 or PA_BF16 (the matrix-core path) */
  pa_dtype out_dtype;          /* PA_F32 or kv_dtype */
  int32_t split_weights;       /* bf16 caches: 0 (default) or 1, see below; else ignored */
} pa_prefill_shape;

/* Queries per prefill work item (one query tile of one sequence). */
#define PA_PREFILL_TILE 128

/*
 * paged_attn_prefill: causal multi-query attention over the paged cache.
 *
 *   q             [T, H, D] in kv_dtype; sequence s owns rows
 *                 query_start[s] .. query_start[s+1]-1
 *   query_start   [S + 1] int32 (device), non-decreasing, query_start[S] <= T
 *   block_tables, context_lens, k_cache, v_cache, block_size, scale: as for
 *                 paged_attn_decode (any finite scale)
 *   out           [T, H, D] in out_dtype
 *   work_order    NULL, or device int32 [S * Tq] with
 *                 Tq = ceil(max_query_len / PA_PREFILL_TILE): the order in
 *                 which the launch's work items are dispatched, a
 *                 permutation of 0 .. S*Tq-1. Item s * Tq + t is query tile t
 *                 of sequence s: its queries t * PA_PREFILL_TILE ..
 *                 (t+1) * PA_PREFILL_TILE - 1, counted from the sequence's
 *                 first query (items past its last query do nothing). Values
 *                 are clamped into range; an item missing from the order
 *                 gets no output. NULL dispatches sequence by sequence, each
 *                 sequence's later tiles first. Items that see the most keys
 *                 first make the launch's tail shorter; prefill_order in the
 *                 Python binding computes that order. Outputs do not depend
 *                 on it.
 *
 * The n_s = query_start[s+1] - query_start[s] queries of sequence s are its
 * last n_s tokens, whose K and V are already in the cache: query r sits at
 * position p = ctx_s - n_s + r and attends to tokens 0 .. p ("Solving the LLM
 * Memory Wall", "1. The Mathematical Foundation": o_i = sum over j <= i of
 * softmax_j(a_ij) v_j). n_s = ctx_s is a whole prompt, n_s < ctx_s a chunk of
 * one, n_s = 1 a decode step. Device-side preconditions: 0 <= n_s <= ctx_s and
 * n_s <= max_query_len (larger values are clamped). Scores and the output
 * accumulate in fp32 on the matrix cores. The weighted sum of V takes fp16
 * operands: each softmax weight rounded once to fp16, a rounding the
 * normaliser also sums, so every output is a convex combination of value
 * rows. bf16 V is converted to fp16 on chip (to nearest), exactly for
 * magnitudes in [2^-14, 2^16); smaller ones are rounded to a multiple of
 * 2^-24. A work item that meets a larger V value, an infinity or a NaN (or
 * non-finite q or k) redoes its tiles as with split_weights = 1. split_weights = 1 (bf16 caches) keeps V in bf16 and
 * enters each weight as a bf16 value plus its bf16 residual, ~16 significant
 * bits, at about 12 % more time. Any other value is PA_EINVAL.
 * S * Tq * H must not exceed 2^31 - 1 (else PA_EINVAL).
 */
pa_status paged_attn_prefill(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             const int32_t* query_start, int32_t block_size, float scale,
                             void* out, const pa_prefill_shape* shape,
                             const int32_t* work_order, void* stream);

/*
 * paged_gather: block translation made visible, for checking it bit for bit.
 * Copies, for each sequence s and token i < context_lens[s], the row
 * cache[block_tables[s][i / B]][i % B] ([H, D], `dtype`) to
 * out[out_row_start[s] + i]. Uses the same device translation routine as
 * paged_attn_decode's general path. out_row_start is a device int64 [S]
 * array chosen by the caller (normally the prefix sums of context_lens).
 * cache and out 16-byte aligned, block_tables and context_lens 4-byte,
 * out_row_start 8-byte (else PA_EALIGN). Not part of the hot path.
 */
pa_status paged_gather(const void* cache, const int32_t* block_tables,
                       const int32_t* context_lens, const int64_t* out_row_start, void* out,
                       int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size,
                       int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                       pa_dtype dtype, void* stream);

/*
 * pa_stream_read: benchmark support, not part of the attention path. Reads
 * `bytes` bytes (a multiple of 16; buf 16-byte aligned, device memory) with
 * the non-temporal 16-byte loads the decode kernel uses and no other work,
 * so its bandwidth is the ceiling those loads can reach on the device.
 * `sink` (device uint32) is written only in a practically impossible case;
 * it keeps the loads from being optimised away. Stamps the launch events of
 * pa_set_launch_events like the attention kernels. bytes == 0 queues
 * nothing.
 */
pa_status pa_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/*
 * pa_frame_read: benchmark support, not part of the attention path. Reads a
 * device buffer of `bytes` bytes holding num_frames frames of frame_bytes
 * each, in the order frame_order (device int32 [num_frames]; entries are
 * clamped into [0, num_frames)), with the decode kernel's non-temporal
 * 16-byte loads and no other work. Frames are read in units of
 * frames_per_unit consecutive entries of frame_order; one workgroup per
 * (group g, unit) reads from each of its frames f the `pieces` pieces of
 * piece_bytes at f * frame_bytes + g * group_stride + p * piece_stride
 * (p < pieces), its 8 wavefronts taking the frames round robin. So the
 * byte pattern of one head's rows in a [NB, B, H, D] cache (group_stride =
 * one row of one head, piece_stride = one token's row of all heads), in a
 * head-major [NB, H, B, D] one (group_stride = B rows, piece_stride = one
 * row), or of whole frames (one group) can be timed on the same bytes
 * ("PagedAttention: Virtual Memory Guide for LLM Inference", "3.
 * PagedAttention CUDA Kernel Execution", shows a K cache split per head and
 * "1. Sizing the Block Dimension" ties the block size to coalescing).
 * Strides, frame_bytes and piece_bytes must be multiples of 16; every piece
 * must lie inside its frame, num_frames * frame_bytes <= bytes, at most
 * 65,535 units (else PA_EINVAL); buf 16-byte aligned (PA_EALIGN). `sink`
 * (device uint32) is written only in a practically impossible case.
 * Stamps the launch events of pa_set_launch_events like pa_stream_read.
 * num_frames == 0 queues nothing.
 */
pa_status pa_frame_read(const void* buf, int64_t bytes, const int32_t* frame_order,
                        int64_t num_frames, int64_t frame_bytes, int32_t groups,
                        int64_t group_stride, int32_t pieces, int64_t piece_stride,
                        int32_t piece_bytes, int32_t frames_per_unit, uint32_t* sink,
                        void* stream);

/*
 * pa_set_launch_events: kernel-accurate timing, for benchmarks and
 * profilers. While set on a thread, every launch that thread makes of the
 * decode partition kernel (paged_attn_decode, paged_attn_decode_partitions;
 * the grouped partition kernel of paged_attn_decode_grouped), of the prefill
 * kernel (paged_attn_prefill) or of pa_stream_read's or pa_frame_read's
 * kernel stamps `start`
 * with the kernel's own start time and `stop` with its end time (hipEvent_t handles
 * owned by the caller, created with timing enabled; either may be NULL).
 * An event plainly recorded on the stream around a launch also counts the
 * dispatch gap before the kernel starts; these do not. Other kernels are
 * unaffected. Pass NULL, NULL to return to plain launches. Never fails.
 */
pa_status pa_set_launch_events(void* start, void* stop);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
