// Paged decode attention for gfx950: a partition pass and a log-sum-exp merge.
// (Kernels and launch templates; paged_decode.hip and paged_decode_<dtype>.hip
// compile them.)
//
// What is computed ("Solving the LLM Memory Wall: A Deep Dive into
// PagedAttention", "1. The Mathematical Foundation"): for sequence s and head
// h, o = sum_i softmax_i(scale * q . k_i) v_i over the sequence's ctx tokens.
// Where k_i and v_i live ("PagedAttention: Virtual Memory Guide for LLM
// Inference", "The Mathematics of Block Translation"): frame
// block_tables[s][i / B], offset i % B, in caches laid out [NB, B, H, D]
// (page 2, "Implementation"). As page 1 ("3. PagedAttention CUDA Kernel
// Execution") asks, the kernel takes the block table itself: no gathered copy.
//
// Work decomposition. One workgroup per (head group, context partition,
// sequence), head fastest so the workgroups in flight together read whole
// frames (all heads of a token are adjacent). A head group is HP adjacent
// heads: one for rows of 256 bytes or more, enough for 256 contiguous bytes
// per token below that (a 64-byte row alone would leave the other half of
// each 128-byte line to another workgroup, and the line would be fetched
// twice). A workgroup runs kNW wavefronts; a short launch (contexts of a
// few chunks) runs two and a wide launch (long contexts) kWideWaves, both
// with twice the heads where that fits (see "Launch forms" below). The
// workgroup's wavefronts take the partition's chunks of kCH tokens round
// robin. Inside a wavefront, each cache row (one token's D
// elements of one head) is spread over kLPR lanes holding 16 bytes each, so
// one load instruction moves kRPL whole rows (kRPL / HP tokens of HP heads)
// and every lane issues 16-byte loads. q . k is a per-lane dot product (packed
// dot2 instructions for 16-bit types) finished by DPP sums inside each group
// of kLPR lanes. Softmax is online: each lane group keeps its own running
// maximum m (in log2 units), sum l and fp32 accumulator for its kVEC output
// elements; groups are combined by cross-lane shuffles, wavefronts through
// LDS, both with the log-sum-exp rule. The context partitions of one
// sequence are combined the same way by the merge kernel.
//
// An optional dispatch order maps the launch's last grid index to the
// sequence (or group) it serves, so that the longest work starts first.
// The grouped pass serves up to four sequences per workgroup whose block
// tables start with the same frames (forks of one prompt): each shared row
// is loaded once and folded into every member's softmax ("PagedAttention:
// Virtual Memory Guide for LLM Inference", "2. Zero-Copy Branching via
// Copy-on-Write", shares the frames; here the reads are shared too).
//
// Masking: tokens at or past ctx are never loaded; their score is -inf and
// their weight exactly 0, so NaN-filled unused slots cannot leak in. The
// running maximum starts at a large finite negative value so that no
// inf - inf ever reaches exp2.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

// No multiply-add contraction beyond the fmaf calls written out: the
// grouped and ungrouped passes inline the same helpers into different code,
// and their results must agree bit for bit.
#pragma clang fp contract(off)

namespace pa {
namespace {

constexpr float kNegBig = -1.0e30f;
constexpr int kNW = 8;          // wavefronts per workgroup of the default form
constexpr int kWideWaves = 16;  // of the wide form (see wide_launch)
constexpr int kU = 4;   // row loads per lane per chunk (for each of K and V)

template <bool kStream>
__device__ __forceinline__ u32x4 load_row(const char* p) {
  if constexpr (kStream)
    return load16_stream(p);
  else
    return load16(p);
}

// A workgroup serves HP adjacent heads. With HP > 1 the lane groups of one
// load take the HP heads in turn, so each token's HP rows (adjacent in a
// [NB, B, H, D] frame) are read as one contiguous span: rows under 256 bytes
// then no longer leave the rest of a 128-byte line to another workgroup.
template <typename T, int D, int HP>
struct Tiling {
  static constexpr int kVEC = Vec<T>::kElems;  // elements a lane holds per row
  static constexpr int kLPR = D / kVEC;        // lanes per cache row
  static constexpr int kRPL = 64 / kLPR;       // rows per wavefront load
  static constexpr int kTPL = kRPL / HP;       // tokens per wavefront load
  static constexpr int kCH = kU * kTPL;        // tokens per chunk
  static_assert(kLPR >= 1 && kLPR <= 64 && (64 % kLPR) == 0, "row must tile a wavefront");
  static_assert(HP >= 1 && kRPL % HP == 0, "a load must hold whole tokens");
};

// Heads per workgroup for a row of `row_bytes`: enough for 256 contiguous
// bytes per token (rows are 32 bytes or more).
constexpr int preferred_heads(int row_bytes) {
  return row_bytes >= 256 ? 1 : 256 / row_bytes;
}

// Per-lane constants of the chunk loads of one (sequence, head group).
template <typename T, int D, int BT, bool kStream, int HP>
struct ChunkLoader {
  using Tl = Tiling<T, D, HP>;
  static constexpr int VEC = Tl::kVEC, LPR = Tl::kLPR, TPL = Tl::kTPL, CH = Tl::kCH;
  // Uniform translation: with a compile-time block size that is a multiple
  // of the tokens per load, the kTPL tokens of one load share a frame, so
  // the frame is read once per load as a scalar.
  static constexpr bool kUniformFrame = BT > 0 && (BT % TPL) == 0;

  const char* kbase;
  const char* vbase;
  // Byte strides of the [NB, B, H, D] caches: one token row (all heads) and
  // one frame. The host guarantees frame_bytes < 2^31, so offsets inside a
  // frame fit 32 bits; frame bases are 64-bit scalars.
  uint32_t row_bytes;
  int64_t frame_bytes;
  uint32_t lane_bytes;  // this lane's 16 bytes inside a token row
  uint32_t max_frame;   // num_blocks - 1 (num_blocks <= 2^31)
  int32_t block_size;
  int64_t num_blocks;
  int tok;              // which of the kTPL tokens of a load this lane reads

  // h0: the group's first head; the lane reads head h0 + (lane / LPR) % HP.
  __device__ __forceinline__ ChunkLoader(const DecodeArgs& a, const int h0, const int lane) {
    kbase = static_cast<const char*>(a.k_cache);
    vbase = static_cast<const char*>(a.v_cache);
    row_bytes = static_cast<uint32_t>(a.num_heads) * D * T::kBytes;
    frame_bytes = static_cast<int64_t>(row_bytes) * a.block_size;
    tok = lane / LPR / HP;
    const uint32_t h = static_cast<uint32_t>(h0 + (lane / LPR) % HP);
    lane_bytes = (h * D + (lane % LPR) * VEC) * T::kBytes;
    max_frame = static_cast<uint32_t>(a.num_blocks - 1);
    block_size = a.block_size;
    num_blocks = a.num_blocks;
  }

  // The chunk of CH tokens starting at t0 (tokens of a sequence whose block
  // table row is table_row): kU row loads of K and of V per lane. kMasked is
  // false for chunks wholly inside [t0, tok_end), which then load without
  // any per-lane condition; masked rows load nothing and are marked invalid.
  template <bool kMasked>
  __device__ __forceinline__ void load(const int32_t* table_row, const int t0, const int tok_end,
                                       u32x4 (&kv)[kU], u32x4 (&vv)[kU], bool (&valid)[kU]) const {
#pragma unroll
    for (int u = 0; u < kU; ++u) valid[u] = !kMasked || (t0 + u * TPL + tok < tok_end);
    if constexpr (kUniformFrame) {
      // All block-table reads of the chunk first (scalar loads). A load
      // wholly past tok_end reads the last valid table entry instead (its
      // rows are masked), so table columns past ceil(ctx / B) are never read.
      uint32_t frame[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t tu = static_cast<uint32_t>(t0 + u * TPL);  // wave-uniform
        const uint32_t tc = kMasked ? min(tu, static_cast<uint32_t>(tok_end - 1)) : tu;
        frame[u] = static_cast<uint32_t>(table_row[tc / BT]);
      }
      int64_t step_base[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t tu = static_cast<uint32_t>(t0 + u * TPL);
        // Out-of-range (or negative) entries are clamped into the pool.
        const uint32_t f = min(frame[u], max_frame);
        step_base[u] = static_cast<int64_t>(f) * frame_bytes + static_cast<int64_t>(tu % BT) * row_bytes;
      }
      const uint32_t lane_off = tok * row_bytes + lane_bytes;
      // Every K row of the chunk is issued before any V row: 1-2 % faster
      // than interleaving K and V row by row. (Not for an earlier start of
      // the scores: a form whose scores begin as each K row arrives, instead
      // of after all eight loads, ran alike.)
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        u32x4 kz = {0u, 0u, 0u, 0u};
        if (valid[u]) kz = load_row<kStream>(kbase + step_base[u] + lane_off);
        kv[u] = kz;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        u32x4 vz = {0u, 0u, 0u, 0u};
        if (valid[u]) vz = load_row<kStream>(vbase + step_base[u] + lane_off);
        vv[u] = vz;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        u32x4 kz = {0u, 0u, 0u, 0u}, vz = {0u, 0u, 0u, 0u};
        if (valid[u]) {
          const int64_t off =
              token_row(table_row, t0 + u * TPL + tok, block_size, num_blocks) * row_bytes +
              lane_bytes;
          kz = load_row<kStream>(kbase + off);
          vz = load_row<kStream>(vbase + off);
        }
        kv[u] = kz;
        vv[u] = vz;
      }
    }
  }
};

// Online-softmax state of one query in one lane group: running maximum m
// (log2 units), running sum l and the lane's kVEC accumulator elements.
template <typename T, int D>
struct SoftmaxState {
  static constexpr int VEC = Tiling<T, D, 1>::kVEC;
  float m, l;
  float acc[VEC];

  __device__ __forceinline__ void reset() {
    m = kNegBig;
    l = 0.f;
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] = 0.f;
  }

  // Fold one loaded chunk into the state: scores q . k (DPP sums inside each
  // lane group), scaled into log2 units; rows marked invalid weigh exactly 0.
  __device__ __forceinline__ void update(const u32x4 qv, const float scale_log2,
                                         const u32x4 (&kv)[kU], const u32x4 (&vv)[kU],
                                         const bool (&valid)[kU]) {
    constexpr int LPR = Tiling<T, D, 1>::kLPR;
    float sc[kU];
    float cmax = kNegBig;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float d = group_sum<LPR>(dot16(T{}, qv, kv[u]));
      sc[u] = valid[u] ? d * scale_log2 : -__builtin_inff();
      cmax = fmaxf(cmax, sc[u]);
    }
    const float m_new = fmaxf(m, cmax);
    const float alpha = fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] *= alpha;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float p = fast_exp2(sc[u] - m_new);
      l += p;
      float vf[VEC];
      widen(T{}, vv[u], vf);
#pragma unroll
      for (int j = 0; j < VEC; ++j) acc[j] = __builtin_fmaf(p, vf[j], acc[j]);
    }
    m = m_new;
  }
};

// LDS of the wavefront combine, sized by the launch for its nw wavefronts
// (dynamic shared memory): per wavefront, each of the HP heads' running
// maximum, sum and accumulator.
template <int D, int HP>
struct CombineLds {
  float* base;
  int nw;
  __device__ __forceinline__ float& m(int w, int hs) const { return base[w * HP + hs]; }
  __device__ __forceinline__ float& l(int w, int hs) const { return base[(nw + w) * HP + hs]; }
  __device__ __forceinline__ float& acc(int w, int e) const {
    return base[2 * nw * HP + w * HP * D + e];
  }
};

template <int D, int HP>
constexpr size_t combine_lds_bytes(int nw) {
  return static_cast<size_t>(nw) * HP * (D + 2) * sizeof(float);
}

extern __shared__ float combine_lds[];

// Combine a (sequence, head group, partition)'s states of all lane groups
// and wavefronts (log-sum-exp rule, for each head apart) and store the
// result: the normalised output when the sequence has one partition, else
// the partition's partial (max, sum, unnormalised output) in the workspace.
// Every thread of the workgroup calls it; it synchronises the workgroup and
// leaves `lds` free for reuse after a further barrier.
template <typename T, int D, int HP>
__device__ __forceinline__ void finish_partition(const DecodeArgs& a, const int s, const int h0,
                                                 const int part, const int n_parts,
                                                 SoftmaxState<T, D> st, const CombineLds<D, HP>& lds) {
  using Tl = Tiling<T, D, HP>;
  constexpr int VEC = Tl::kVEC, LPR = Tl::kLPR;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = a.waves;  // the launch's choice, 2..kWideWaves
  const int lane = threadIdx.x & 63;
  const int grp = lane / LPR;
  const int col = lane % LPR;
  float m = st.m, l = st.l;
  // Combine the lane groups of the wavefront that hold the same head (lanes
  // col + LPR * (head + HP * i)).
#pragma unroll
  for (int x = LPR * HP; x < 64; x <<= 1) {
    const float m_o = __shfl_xor(m, x);
    const float l_o = __shfl_xor(l, x);
    const float m_n = fmaxf(m, m_o);
    const float fa = fast_exp2(m - m_n);
    const float fb = fast_exp2(m_o - m_n);
    l = __builtin_fmaf(l, fa, l_o * fb);
#pragma unroll
    for (int j = 0; j < VEC; ++j)
      st.acc[j] = __builtin_fmaf(st.acc[j], fa, __shfl_xor(st.acc[j], x) * fb);
    m = m_n;
  }

  // Combine the wavefronts through LDS.
  if (grp < HP) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) lds.acc(wave, grp * D + col * VEC + j) = st.acc[j];
    if (col == 0) {
      lds.m(wave, grp) = m;
      lds.l(wave, grp) = l;
    }
  }
  __syncthreads();

  for (int e = threadIdx.x; e < HP * D; e += nw * 64) {
    const int hs = e / D;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < kWideWaves; ++w)
      if (w < nw) M = fmaxf(M, lds.m(w, hs));
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWideWaves; ++w) {
      if (w >= nw) break;
      const float fw = fast_exp2(lds.m(w, hs) - M);
      L = __builtin_fmaf(lds.l(w, hs), fw, L);
      O = __builtin_fmaf(lds.acc(w, e), fw, O);
    }
    const int64_t sh = static_cast<int64_t>(s) * a.num_heads + h0 + hs;
    const int el = e - hs * D;
    if (n_parts == 1) {
      const float r = L > 0.f ? O / L : 0.f;
      const int64_t o = sh * D + el;
      if constexpr (T::kBytes == 4) {
        static_cast<float*>(a.out)[o] = r;
      } else {
        if (a.out_f32)
          static_cast<float*>(a.out)[o] = r;
        else
          static_cast<uint16_t*>(a.out)[o] = static_cast<uint16_t>(narrow_bits(T{}, r));
      }
    } else {
      const int64_t p = sh * a.max_parts + part;
      a.ws_acc[p * D + el] = O;
      if (el == 0) {
        a.ws_ml[2 * p] = M;
        a.ws_ml[2 * p + 1] = L;
      }
    }
  }
}

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, const int s) {
  const int ctx = a.context_lens[s];
  return ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
}

__device__ __forceinline__ int parts_of(const DecodeArgs& a, const int ctx) {
  return ctx <= a.part_tokens ? 1 : (ctx + a.part_tokens - 1) / a.part_tokens;
}

// kStream selects non-temporal K/V loads (frames read once) or ordinary
// cached loads (frames shared by several sequences of the call).
// Eight wavefronts per SIMD (at most 64 registers per lane): the kernel is
// bound by memory latency, so it keeps the most loads in flight.
template <typename T, int D, int BT, bool kStream, int HP>
__global__ __launch_bounds__(kWideWaves * 64) __attribute__((amdgpu_waves_per_eu(8)))
void decode_partition_kernel(DecodeArgs a) {
  using Ld = ChunkLoader<T, D, BT, kStream, HP>;
  constexpr int VEC = Ld::VEC, LPR = Ld::LPR, CH = Ld::CH;

  const int h0 = blockIdx.x * HP;
  const int part = blockIdx.y;
  const int s = a.seq_order ? min(max(a.seq_order[blockIdx.z], 0), a.num_seqs - 1)
                            : static_cast<int>(blockIdx.z);
  const int ctx = clamp_ctx(a, s);
  const int n_parts = parts_of(a, ctx);
  if (part >= n_parts) return;  // uniform over the workgroup
  const int tok_begin = part * a.part_tokens;
  const int tok_end = min(ctx, tok_begin + a.part_tokens);

  // readfirstlane tells the compiler the wavefront index is uniform, so the
  // chunk loop, block-table reads and frame arithmetic stay scalar.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const Ld ld(a, h0, lane);
  const int32_t* table_row = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;
  const int h = h0 + (lane / LPR) % HP;  // this lane's head
  const u32x4 qv = load16(static_cast<const char*>(a.q) +
                          ((static_cast<int64_t>(s) * a.num_heads + h) * D + (lane % LPR) * VEC) *
                              T::kBytes);

  SoftmaxState<T, D> st;
  st.reset();
  const int nw = a.waves;  // the launch's choice, 2..kWideWaves
  const int n_chunks = (tok_end - tok_begin + CH - 1) / CH;
  for (int chunk = wave; chunk < n_chunks; chunk += nw) {
    const int t0 = tok_begin + chunk * CH;
    u32x4 kv[kU], vv[kU];
    bool valid[kU];
    if (t0 + CH <= tok_end) {
      ld.template load<false>(table_row, t0, tok_end, kv, vv, valid);
    } else {
      ld.template load<true>(table_row, t0, tok_end, kv, vv, valid);
    }
    st.update(qv, a.scale_log2, kv, vv, valid);
  }

  const CombineLds<D, HP> lds{combine_lds, nw};
  finish_partition<T, D, HP>(a, s, h0, part, n_parts, st, lds);
}

// Grouped partition pass: a workgroup serves a group of up to G sequences
// (batch indices group_start[g] .. group_start[g + 1] - 1) whose block
// tables agree on the first group_shared[g] tokens. Partition p covers the
// same tokens [p * P, (p + 1) * P) as in the ungrouped pass. Chunks below
// the shared length are loaded once and folded into every member's state;
// the remaining chunks are each member's own. Chunk boundaries and the
// chunk-to-wavefront assignment are those of the ungrouped pass (the shared
// length is rounded down to a whole chunk), so every member's result equals
// the ungrouped pass's bit for bit.
template <typename T, int D, int BT, bool kStream, int HP, int G>
__global__ __launch_bounds__(kWideWaves * 64) void decode_group_kernel(DecodeArgs a, GroupArgs g) {
  using Ld = ChunkLoader<T, D, BT, kStream, HP>;
  constexpr int VEC = Ld::VEC, LPR = Ld::LPR, CH = Ld::CH;

  const int h0 = blockIdx.x * HP;
  const int part = blockIdx.y;
  const int gi = a.seq_order ? min(max(a.seq_order[blockIdx.z], 0), g.num_groups - 1)
                             : static_cast<int>(blockIdx.z);
  const int s0 = min(max(g.group_start[gi], 0), a.num_seqs);
  const int ns = min(max(g.group_start[gi + 1], s0), a.num_seqs) - s0;  // members (<= G)
  const int members = min(ns, G);
  int ctx[G];
  int max_ctx = 0, min_ctx = a.max_ctx;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    ctx[i] = i < members ? clamp_ctx(a, s0 + i) : 0;
    if (i < members) {
      max_ctx = max(max_ctx, ctx[i]);
      min_ctx = min(min_ctx, ctx[i]);
    }
  }
  if (members == 0 || part >= parts_of(a, max_ctx)) return;  // uniform over the workgroup
  const int tok_begin = part * a.part_tokens;
  // shared tokens: at most every member's context, whole chunks only
  int shared = min(g.group_shared[gi], min_ctx);
  shared = shared < 0 ? 0 : shared / CH * CH;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = a.waves;  // the launch's choice, 2..kWideWaves
  const int lane = threadIdx.x & 63;
  const Ld ld(a, h0, lane);
  const int h = h0 + (lane / LPR) % HP;  // this lane's head

  u32x4 qv[G];
  SoftmaxState<T, D> st[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    st[i].reset();
    qv[i] = u32x4{0u, 0u, 0u, 0u};
    if (i < members)
      qv[i] = load16(static_cast<const char*>(a.q) +
                     ((static_cast<int64_t>(s0 + i) * a.num_heads + h) * D + (lane % LPR) * VEC) *
                         T::kBytes);
  }

  // Shared chunks: [tok_begin, sh_end), every one whole and inside every
  // member's context; the first member's table row addresses them.
  const int sh_end = min(shared, tok_begin + a.part_tokens);
  const int n_shared = sh_end > tok_begin ? (sh_end - tok_begin) / CH : 0;
  const int32_t* row0 = a.block_tables + static_cast<int64_t>(s0) * a.max_blocks;
  for (int chunk = wave; chunk < n_shared; chunk += nw) {
    const int t0 = tok_begin + chunk * CH;
    u32x4 kv[kU], vv[kU];
    bool valid[kU];
    ld.template load<false>(row0, t0, sh_end, kv, vv, valid);
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (i < members) st[i].update(qv[i], a.scale_log2, kv, vv, valid);
  }

  // Each member's own chunks, numbered on from the shared ones so that
  // wavefront w keeps every chunk c with c % nw == w.
#pragma unroll
  for (int i = 0; i < G; ++i) {
    if (i >= members) break;
    const int tok_end = min(ctx[i], tok_begin + a.part_tokens);
    const int n_chunks = tok_end > tok_begin ? (tok_end - tok_begin + CH - 1) / CH : 0;
    const int32_t* row = a.block_tables + static_cast<int64_t>(s0 + i) * a.max_blocks;
    int chunk = n_shared + ((wave - n_shared) % nw + nw) % nw;
    for (; chunk < n_chunks; chunk += nw) {
      const int t0 = tok_begin + chunk * CH;
      u32x4 kv[kU], vv[kU];
      bool valid[kU];
      if (t0 + CH <= tok_end) {
        ld.template load<false>(row, t0, tok_end, kv, vv, valid);
      } else {
        ld.template load<true>(row, t0, tok_end, kv, vv, valid);
      }
      st[i].update(qv[i], a.scale_log2, kv, vv, valid);
    }
  }

  const CombineLds<D, HP> lds{combine_lds, nw};
#pragma unroll
  for (int i = 0; i < G; ++i) {
    if (i >= members) break;
    const int n_parts = parts_of(a, ctx[i]);
    if (part < n_parts) {  // uniform: the member has tokens in this partition
      finish_partition<T, D, HP>(a, s0 + i, h0, part, n_parts, st[i], lds);
      __syncthreads();  // lds is reused by the next member
    }
  }
}

// Log-sum-exp merge of a sequence's partitions: with M = max_p m_p,
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p. The workgroup
// reduces the partitions' maxima and normalisers in parallel; for the
// weighted sum wavefront w takes partitions w, w + kMergeWaves, ..., in
// groups of kMergeUnroll whose rows are all loaded before they are summed
// (the first group before the maximum is known), and the wavefronts' parts
// are added in LDS. The order of every sum is fixed by the launch shape, so
// results repeat bit for bit.
constexpr int kMergeWaves = 2;
constexpr int kMergeUnroll = 8;
constexpr int kMergeChunk = 1024;  // partitions whose weights sit in LDS at a time
static_assert(kMergeChunk % (kMergeWaves * kMergeUnroll) == 0, "groups must not straddle chunks");

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

template <typename T, int D>
__global__ __launch_bounds__(kMergeWaves * 64) void decode_merge_kernel(DecodeArgs a) {
  constexpr int kEPL = (D + 63) / 64;  // output elements per lane
  __shared__ float red_max[kMergeWaves], red_sum[kMergeWaves];
  __shared__ float weights[kMergeChunk];
  __shared__ float parts[kMergeWaves][D];
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  int n_parts = ctx <= a.part_tokens ? 1 : (ctx + a.part_tokens - 1) / a.part_tokens;
  if (n_parts <= 1) return;  // written by the partition pass
  n_parts = min(n_parts, a.max_parts);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t sh = static_cast<int64_t>(s) * a.num_heads + h;
  const float* ml = a.ws_ml + 2 * sh * a.max_parts;
  const float* pacc = a.ws_acc + sh * a.max_parts * D;

  // rows of the group of partitions p0 + u * kMergeWaves (u < kMergeUnroll)
  float rows[kMergeUnroll][kEPL];
  auto load_rows = [&](const int p0) {
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int p = p0 + u * kMergeWaves;
#pragma unroll
      for (int k = 0; k < kEPL; ++k) {
        const int e = lane + 64 * k;
        rows[u][k] = (p < n_parts && e < D) ? pacc[static_cast<int64_t>(p) * D + e] : 0.f;
      }
    }
  };
  load_rows(wave);

  float mx = kNegBig;
  for (int p = tid; p < n_parts; p += kMergeWaves * 64) mx = fmaxf(mx, ml[2 * p]);
  mx = wave_max(mx);
  if (lane == 0) red_max[wave] = mx;
  __syncthreads();
  float M = red_max[0];
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, red_max[w]);

  float L = 0.f;
  float O[kEPL];
#pragma unroll
  for (int k = 0; k < kEPL; ++k) O[k] = 0.f;
  for (int c0 = 0; c0 < n_parts; c0 += kMergeChunk) {
    const int cn = min(kMergeChunk, n_parts - c0);
    __syncthreads();  // the previous chunk's weights are no longer read
    for (int p = tid; p < cn; p += kMergeWaves * 64) {
      const float f = fast_exp2(ml[2 * (c0 + p)] - M);
      weights[p] = f;
      L += ml[2 * (c0 + p) + 1] * f;
    }
    __syncthreads();
    for (int p0 = wave; p0 < cn; p0 += kMergeWaves * kMergeUnroll) {
      if (c0 + p0 != wave) load_rows(c0 + p0);  // the first group is loaded
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        const int p = p0 + u * kMergeWaves;
        if (p < cn) {
          const float f = weights[p];
#pragma unroll
          for (int k = 0; k < kEPL; ++k) O[k] = __builtin_fmaf(rows[u][k], f, O[k]);
        }
      }
    }
  }
  L = wave_sum(L);
  if (lane == 0) red_sum[wave] = L;
#pragma unroll
  for (int k = 0; k < kEPL; ++k) {
    const int e = lane + 64 * k;
    if (e < D) parts[wave][e] = O[k];
  }
  __syncthreads();
  float Lt = red_sum[0];
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) Lt += red_sum[w];
  for (int e = tid; e < D; e += kMergeWaves * 64) {
    float o = parts[0][e];
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) o += parts[w][e];
    const float r = Lt > 0.f ? o / Lt : 0.f;
    const int64_t oi = sh * D + e;
    if constexpr (T::kBytes == 4) {
      static_cast<float*>(a.out)[oi] = r;
    } else {
      if (a.out_f32)
        static_cast<float*>(a.out)[oi] = r;
      else
        static_cast<uint16_t*>(a.out)[oi] = static_cast<uint16_t>(narrow_bits(T{}, r));
    }
  }
}

// Heads per workgroup of a launch: the preferred grouping for the row size,
// halved until it divides the head count.
inline int heads_per_group(int row_bytes, int num_heads) {
  int hp = preferred_heads(row_bytes);
  while (hp > 1 && num_heads % hp != 0) hp /= 2;
  return hp;
}

// Launch forms. The default form runs kNW wavefronts on HP heads (the
// row's preferred grouping). Two others serve twice the heads where that
// grouping fits (2 HP divides H and the rows per load), so each token's rows
// of the group form a span twice as long:
//
// Short launches. With kNW wavefronts sharing a context of a few chunks,
// most of them only wait at the combine. When no context exceeds
// kShortChunks chunks (by max_ctx) and the launch has enough workgroups to
// fill the chip at two wavefronts each, a workgroup runs two wavefronts
// (and 2 HP heads if the halved grid still has that many workgroups), so the
// per-workgroup work (prologue, combine, store) covers more rows. Measured
// at 2048 sequences of up to 128 bf16 tokens, d = 128: 438 us with eight
// wavefronts and one head, 396 us with two wavefronts, 376 us with two
// wavefronts and two heads; 512 sequences of up to 512 tokens: 351 and 338
// us; 1024 sequences of up to 1024 tokens: 1354 and 1334 us.
//
// Wide launches: kWideWaves wavefronts on 2 HP heads, the same wavefronts in
// flight as the default form over half the workgroups, when contexts reach
// kWideMinContext tokens in partitions of at least that length, the launch
// has one partition or at least kWideMinParts (two or three partitions, the
// second of them short, ran 4-11% slower than the default form), and the
// grid keeps kWideMinWorkgroups workgroups. Measured against the default
// form: batch 64 x 2048 bf16 tokens 181.5 -> 175.4 us, 8 x 32k 832 -> 794
// us, batch 256 at 64 heads 1701 -> 1613 us, 1024 x 2048 2663 -> 2608 us,
// d = 16 and 64 3.5%; rows of 512 bytes (d = 256 bf16, d = 128 fp32) run
// alike in both forms. The grouped pass of the shared-prefix workload
// (contexts up to about 1200 tokens) keeps the default form: there the wide
// form was 5.5% slower.
//
// Chunks of a doubled grouping are half as long, so partition sizes rounded
// to whole chunks of the default grouping stay whole. The grouped pass makes
// the same choice from the same figures, which keeps its results equal to
// the ungrouped pass's.
constexpr int kShortChunks = 64;
constexpr int64_t kShortMinWorkgroups = 4096;
constexpr int kWideMinContext = 1536;
constexpr int kWideMinParts = 4;
constexpr int64_t kWideMinWorkgroups = 1024;

inline int64_t launch_workgroups(const DecodeArgs& a, int hp) {
  return static_cast<int64_t>(a.num_seqs) * (a.num_heads / hp) * a.max_parts;
}

inline bool short_launch(const DecodeArgs& a, int chunk, int hp) {
  return static_cast<int64_t>(a.max_ctx) <= static_cast<int64_t>(kShortChunks) * chunk &&
         launch_workgroups(a, hp) >= kShortMinWorkgroups;
}

// hp2: the doubled grouping (which must fit).
inline bool wide_launch(const DecodeArgs& a, int hp2) {
  return a.max_ctx >= kWideMinContext && a.part_tokens >= kWideMinContext &&
         (a.max_parts == 1 || a.max_parts >= kWideMinParts) &&
         launch_workgroups(a, hp2) >= kWideMinWorkgroups;
}

// Ungrouped (g == nullptr) or grouped partition pass, HP heads and `waves`
// wavefronts per workgroup.
template <typename T, int D, int BT, int HP>
hipError_t launch_part(const DecodeArgs& args, const GroupArgs* g, int waves, hipStream_t stream) {
  DecodeArgs a = args;
  a.waves = waves;
  const dim3 block(a.waves * 64);
  const size_t lds = combine_lds_bytes<D, HP>(waves);
  if (g != nullptr) {
    const dim3 grid(a.num_heads / HP, a.max_parts, g->num_groups);
    if (a.stream_loads)
      return launch_timed_lds(decode_group_kernel<T, D, BT, true, HP, kMaxGroup>, grid, block, lds,
                              stream, a, *g);
    return launch_timed_lds(decode_group_kernel<T, D, BT, false, HP, kMaxGroup>, grid, block, lds,
                            stream, a, *g);
  }
  const dim3 grid(a.num_heads / HP, a.max_parts, a.num_seqs);
  if (a.stream_loads)
    return launch_timed_lds(decode_partition_kernel<T, D, BT, true, HP>, grid, block, lds, stream, a);
  return launch_timed_lds(decode_partition_kernel<T, D, BT, false, HP>, grid, block, lds, stream, a);
}

// HP heads per workgroup (the row's preferred grouping, halved until it
// divides H; every such grouping is compiled) in the default form, or the
// short or wide form with 2 HP heads where that grouping fits.
template <typename T, int D, int BT, int HP = preferred_heads(D * T::kBytes)>
hipError_t launch_heads(const DecodeArgs& a, const GroupArgs* g, hipStream_t stream) {
  if constexpr (HP > 1) {
    if (a.num_heads % HP != 0) return launch_heads<T, D, BT, HP / 2>(a, g, stream);
  }
  constexpr bool kDoubles = Tiling<T, D, 1>::kRPL % (2 * HP) == 0;
  const bool doubles = kDoubles && a.num_heads % (2 * HP) == 0;
  if (short_launch(a, Tiling<T, D, HP>::kCH, HP)) {
    if constexpr (kDoubles) {
      if (doubles && launch_workgroups(a, 2 * HP) >= kShortMinWorkgroups)
        return launch_part<T, D, BT, 2 * HP>(a, g, 2, stream);
    }
    return launch_part<T, D, BT, HP>(a, g, 2, stream);
  }
  if constexpr (kDoubles) {
    if (doubles && wide_launch(a, 2 * HP)) return launch_part<T, D, BT, 2 * HP>(a, g, kWideWaves, stream);
  }
  return launch_part<T, D, BT, HP>(a, g, kNW, stream);
}

// Block sizes with a uniform-frame specialisation (a multiple of the rows
// of one load, so of the tokens of one load for any head grouping); other
// sizes take the per-lane translation path (BT = 0).
template <typename T, int D>
hipError_t dispatch_block(const DecodeArgs& a, const GroupArgs* g, hipStream_t stream) {
  constexpr int RPL = Tiling<T, D, 1>::kRPL;
  switch (a.block_size) {
    case 8:
      if constexpr (8 % RPL == 0) return launch_heads<T, D, 8>(a, g, stream);
      break;
    case 16:
      if constexpr (16 % RPL == 0) return launch_heads<T, D, 16>(a, g, stream);
      break;
    case 32:
      if constexpr (32 % RPL == 0) return launch_heads<T, D, 32>(a, g, stream);
      break;
    case 64:
      if constexpr (64 % RPL == 0) return launch_heads<T, D, 64>(a, g, stream);
      break;
    default:
      break;
  }
  return launch_heads<T, D, 0>(a, g, stream);
}

template <typename T>
hipError_t dispatch_dim(const DecodeArgs& a, const GroupArgs* g, int head_dim,
                        hipStream_t stream) {
  switch (head_dim) {
    case 16: return dispatch_block<T, 16>(a, g, stream);
    case 32: return dispatch_block<T, 32>(a, g, stream);
    case 64: return dispatch_block<T, 64>(a, g, stream);
    case 128: return dispatch_block<T, 128>(a, g, stream);
    case 256: return dispatch_block<T, 256>(a, g, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
hipError_t launch_merge_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.num_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), grid, dim3(kMergeWaves * 64), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t merge_dim(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 16: return launch_merge_t<T, 16>(a, stream);
    case 32: return launch_merge_t<T, 32>(a, stream);
    case 64: return launch_merge_t<T, 64>(a, stream);
    case 128: return launch_merge_t<T, 128>(a, stream);
    case 256: return launch_merge_t<T, 256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// The partition pass (ungrouped with g == nullptr, else grouped) for one
// cache dtype; each is compiled in a file of its own.
hipError_t decode_dispatch_f32(const DecodeArgs& a, const GroupArgs* g, int head_dim,
                               hipStream_t stream);
hipError_t decode_dispatch_f16(const DecodeArgs& a, const GroupArgs* g, int head_dim,
                               hipStream_t stream);
hipError_t decode_dispatch_bf16(const DecodeArgs& a, const GroupArgs* g, int head_dim,
                                hipStream_t stream);

}  // namespace pa
