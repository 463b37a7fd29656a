/*
 * paged_blocks.h - C ABI of the host block manager (frame pool, block tables,
 * slot mapping, copy-on-write, prefix caching). Host code only: no device
 * memory, no stream; every pointer here is a HOST pointer.
 *
 * Rules followed (by page title and section):
 *   - "PagedAttention: Virtual Memory Guide for LLM Inference", "1. Demand
 *     Paging during Autoregressive Decoding" and "Reference Implementation:
 *     Block Table & Paged Cache Manager": free frames are handed out first in,
 *     first out, and a frame whose reference count falls to zero rejoins the
 *     tail of the free list; a prompt of L tokens takes ceil(L / B) frames;
 *     appending token t (t = tokens the sequence holds) takes a new frame
 *     exactly when t mod B == 0, else writes offset t mod B of the last frame.
 *   - Same page, "2. Zero-Copy Branching via Copy-on-Write": a fork shares
 *     every frame and adds a reference to each; appending into a shared
 *     partial last frame first moves the sequence to a private copy of it.
 *   - Same page, "2. Native Synergy with RadixAttention and Prompt Caching",
 *     and "Solving the LLM Memory Wall: A Deep Dive into PagedAttention",
 *     algorithmic step 5: a filled block never changes, so a request whose
 *     prompt starts with the same tokens can use the frames already holding
 *     them.
 *
 * Prefix caching (only for a manager created with prefix_caching != 0):
 *   - a full block is keyed by a 128-bit chain hash of its token ids and the
 *     key of the block before it, so a key names the whole token prefix
 *     that the block completes;
 *   - a block enters the cache when it fills (a prompt's full blocks at
 *     request start; a generated token's block when that token completes
 *     it); the cache holds one reference on each frame it keeps; if the key
 *     is cached already the new frame stays private and nothing changes;
 *   - a new request reuses the longest run of its leading full blocks whose
 *     keys are cached, stopping at the first miss; the partial last block is
 *     never shared;
 *   - each cached frame has a last-use time (entry or reuse: one counter; a
 *     request's reuses in block order, then its new entries in block order);
 *     when the free list is empty the cached frame referenced by the cache
 *     alone with the oldest last use is dropped and freed, then allocation
 *     proceeds;
 *   - a request that cannot get all its frames takes none and changes
 *     nothing.
 *
 * Slots are frame * B + offset: the row index of a [num_frames, B, H, D]
 * cache viewed as [num_frames * B, H, D].
 *
 * Sequence ids are arbitrary int64 values chosen by the caller. A manager is
 * not thread-safe: calls on one manager must not overlap. Every function
 * returns a pb_status; on any error nothing has changed.
 */
#ifndef PAGED_BLOCKS_H
#define PAGED_BLOCKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pb_status {
  PB_OK = 0,
  PB_EINVAL = -1,   /* bad argument: null pointer, negative size, unknown or duplicate id */
  PB_ENOMEM = -2,   /* the pool cannot supply the frames the call needs */
  PB_ESTATE = -3,   /* the call does not fit the manager (e.g. a prefix-cache call
                       on a manager created without prefix caching) */
} pb_status;

typedef struct pb_manager pb_manager;

/* Statistics of a manager. */
typedef struct pb_stats {
  int64_t free_frames;    /* frames on the free list */
  int64_t cached_frames;  /* frames held by the prefix cache */
  int64_t hit_blocks;     /* full blocks reused by requests */
  int64_t miss_blocks;    /* blocks requests had to allocate */
  int64_t evictions;      /* cached frames dropped to refill the free list */
  int64_t sequences;      /* live sequences */
} pb_stats;

/*
 * Create a manager over num_frames frames of block_size tokens. `order`
 * (num_frames int32 values, a permutation of 0 .. num_frames-1, or NULL for
 * ascending) is the initial free list, head first. prefix_caching != 0
 * enables the prefix cache. *out receives the manager (owned by the caller;
 * release it with pb_destroy).
 */
pb_status pb_create(int64_t num_frames, int32_t block_size, const int32_t* order,
                    int32_t prefix_caching, pb_manager** out);
void pb_destroy(pb_manager* m);

/*
 * Start sequence `sid` with a prompt of n_tokens tokens: ceil(n / B) frames
 * at once, first in first out. slots_out (n_tokens int64, may be NULL when
 * n_tokens == 0) receives the slot of every position. No prefix reuse.
 */
pb_status pb_init_sequence(pb_manager* m, int64_t sid, int64_t n_tokens, int64_t* slots_out);

/*
 * Start request `sid` with prompt token ids tokens[0 .. n). With prefix
 * caching the leading cached full blocks are reused: *reused_out receives
 * the number of leading positions whose K/V is already in the cache (a
 * multiple of B); positions from there on must be written. slots_out (n
 * int64) receives the slot of every position, reused or not. Without prefix
 * caching this is pb_init_sequence and *reused_out is 0.
 */
pb_status pb_init_sequence_tokens(pb_manager* m, int64_t sid, const int64_t* tokens, int64_t n,
                                  int64_t* reused_out, int64_t* slots_out);

/*
 * Append one token to each of n sequences, in order (a sequence may appear
 * more than once). token_ids (n values) are the tokens' ids for the prefix
 * cache, or NULL (then no block completed here enters the cache).
 * slots_out[i] receives the slot of token i. cow_out (n * 3 int64, may be
 * NULL) receives for token i either (-1, -1, 0) or, when the append moved
 * the sequence to a private copy of a shared partial frame, (source frame,
 * new frame, rows to copy): the caller copies those rows, offsets
 * 0 .. rows-1, before writing the token. On PB_ENOMEM the tokens before the
 * failing one have been appended (their outputs are filled) and the failing
 * one and those after it have not; *done_out (may be NULL) receives how many
 * were appended.
 */
pb_status pb_append_tokens(pb_manager* m, const int64_t* sids, const int64_t* token_ids, int64_t n,
                           int64_t* slots_out, int64_t* cow_out, int64_t* done_out);

/* Fork: `child` shares every frame of `parent` (one more reference each). */
pb_status pb_fork(pb_manager* m, int64_t parent, int64_t child);

/* Release a sequence's frames (one reference each); unknown ids are ignored. */
pb_status pb_free_sequence(pb_manager* m, int64_t sid);

/*
 * Block tables of n sequences as an int32 [n, max_blocks] array (unused
 * columns = pad) and their context lengths (int32 [n], may be NULL).
 * PB_EINVAL if a table is longer than max_blocks or an id is unknown.
 */
pb_status pb_block_tables(const pb_manager* m, const int64_t* sids, int64_t n, int32_t pad,
                          int32_t max_blocks, int32_t* tables_out, int32_t* lens_out);

/* Number of frames in a sequence's table (*out), for sizing max_blocks. */
pb_status pb_table_length(const pb_manager* m, int64_t sid, int64_t* out);

/* Free list, head first: up to cap frames into out; *count_out = its length. */
pb_status pb_free_list(const pb_manager* m, int32_t* out, int64_t cap, int64_t* count_out);

/* Reference count of every frame (num_frames int32 values). */
pb_status pb_ref_counts(const pb_manager* m, int32_t* out);

pb_status pb_get_stats(const pb_manager* m, pb_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_BLOCKS_H */
