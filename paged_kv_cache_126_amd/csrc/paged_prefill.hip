// Paged prefill for gfx950: causal multi-query attention over the paged cache
// on the matrix cores.
//
// What is computed ("Solving the LLM Memory Wall: A Deep Dive into
// PagedAttention", "1. The Mathematical Foundation"): query i attends to keys
// j <= i, o_i = sum_{j <= i} softmax_j(q_i . k_j * scale) v_j. The queries of
// sequence s are its last n_s tokens (their K/V already appended), so the
// same kernel serves a whole prompt (n_s = ctx_s) and a chunk of one. Keys
// and values are fetched through the block table ("PagedAttention: Virtual
// Memory Guide for LLM Inference", "The Mathematics of Block Translation").
//
// Work decomposition. One workgroup per (query tile of 128, head, sequence);
// a (sequence, query tile) pair is a work item, dispatched in the caller's
// order, and with H a multiple of 8 head h of every item runs on XCD h % 8.
// Each of the 4
// wavefronts owns 32 consecutive queries. The workgroup walks the keys in
// tiles of 32: the tile's K and V rows are staged in LDS row-major,
// double-buffered (the next tile is fetched into registers meanwhile), then
// every wavefront
//   1. forms S^T = K Q^T (32 keys x 32 queries) with D/16 MFMA 32x32x16
//      steps; Q^T stays in registers as the B operand, so each lane owns one
//      query column and 16 of the tile's keys. The K rows enter in a
//      permuted order chosen so that those 16 keys come out in the B-operand
//      layout of step 3,
//   2. applies the causal mask and an online softmax per query (the two
//      lanes sharing a query exchange one value for the maximum; each keeps
//      its own share of the normaliser, added once at the end),
//   3. accumulates O^T += V^T P^T on fp16 operands: P rounded once to fp16
//      (11 significant bits of every softmax weight; the normaliser sums the
//      rounded weights), and, for bf16 caches, V converted to fp16 (to
//      nearest) as it is staged, which is exact for magnitudes in
//      [2^-14, 2^16); smaller ones are rounded to a multiple of 2^-24. A
//      larger value becomes an fp16 infinity, which makes the accumulators
//      of every wavefront that reads its tile infinite or NaN (inf x 0 for
//      a masked key); a workgroup whose accumulators end non-finite redoes
//      its tiles on bf16 operands with P split into a high part and the
//      residual (two MFMAs, ~16 significant bits); callers can ask for that
//      form throughout.
// Matrix layouts (verified on the device): for v_mfma_f32_32x32x16, A[i][k]
// sits in lane i + 32 * (k / 8), element k % 8; B[k][j] in lane
// j + 32 * (k / 8), element k % 8; D[i][j] in lane j + 32 * ((i / 4) % 2),
// element (i % 4) + 4 * (i / 8).
#include <type_traits>

#include "pa_device.h"
#include "pa_prefill.h"

namespace pa {
namespace {

constexpr int kWaves = 4;                 // wavefronts per workgroup
constexpr int kQW = 32;                   // queries per wavefront
constexpr int kBM = kWaves * kQW;         // queries per workgroup
static_assert(kBM == kPrefillTile, "a work item is one workgroup's query tile");
constexpr int kBN = 32;                   // keys per tile
constexpr float kNegBig = -1.0e30f;
constexpr float kLazy = 8.0f;             // reference-maximum slack, log2 units
constexpr int kTableCache = 2048;         // block-table entries staged in LDS

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 64-bit transposing LDS read (ds_read_b64_tr_b16) of 16-bit elements.
__device__ __forceinline__ v4i16 tr_read(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((__attribute__((address_space(3))) uint16_t*)(p)));
}

// v_permlane32_swap: returns (a's lower half | b's lower half, a's upper
// half | b's upper half), halves being lanes 0-31 and 32-63.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Combine a value with the same lane's value in the other half of the
// wavefront (lane l and l ^ 32): both results are bit-identical.
__device__ __forceinline__ float max_halves(float v) {
  float a = v, b = v;
  swap_halves(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_halves(float v) {
  float a = v, b = v;
  swap_halves(a, b);
  return a + b;
}

__device__ __forceinline__ u32x4 join(v4i16 a, v4i16 b) {
  const uint2 x = __builtin_bit_cast(uint2, a);
  const uint2 y = __builtin_bit_cast(uint2, b);
  return u32x4{x.x, x.y, y.x, y.y};
}

template <typename T>
struct Mfma;

typedef float f32x2 __attribute__((ext_vector_type(2)));

template <>
struct Mfma<BF16> {
  using vec = bf16x8;
  using pair = __bf16 __attribute__((ext_vector_type(2)));  // two weights, rounded together
  static __device__ __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec from_bits(u32x4 v) { return __builtin_bit_cast(vec, v); }
};

template <>
struct Mfma<F16> {
  using vec = f16x8;
  using pair = _Float16 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec from_bits(u32x4 v) { return __builtin_bit_cast(vec, v); }
};

constexpr int kXcds = 8;  // accelerator complex dies of the MI355X

// Three wavefronts per SIMD (at most 168 registers per lane): the tile loop
// fits without spilling once the accumulators live in the general register
// file, and the third wavefront hides the LDS and global-load latency. (The
// bf16 form, which holds both passes, keeps the 64-bit query row offset in
// scratch between its prologue and its epilogue.)
template <typename T, int D>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(3)))
void prefill_kernel(PrefillArgs a) {
  using M = Mfma<T>;
  using vec = typename M::vec;
  constexpr int kSteps = D / 16;   // MFMA k-steps over the head dimension
  constexpr int kDBlk = D / 32;    // 32-row blocks of O^T
  constexpr int kPieces = D / 8;   // 16-byte pieces per cache row
  constexpr int kPadK = 8;         // LDS row padding (elements) against bank conflicts
  constexpr int kPadV = 16;
  constexpr bool kBf16 = std::is_same<T, BF16>::value;

  // Work item and head of this workgroup. Workgroups go to the 8 XCDs
  // round-robin by linear id, and each XCD has its own L2. With H a
  // multiple of 8, head h runs on XCD h % 8 for every item, so the query
  // tiles of one (head, sequence), which read the same keys, share an L2;
  // each XCD takes the items in dispatch order, its H / 8 heads of an item
  // back to back.
  const int ntiles = (a.max_query_len + kBM - 1) / kBM;
  const int nitems = a.num_seqs * ntiles;
  const int lin = static_cast<int>(blockIdx.x);
  int item, h;
  if (a.num_heads % kXcds == 0) {
    const int per = a.num_heads / kXcds;
    const int idx = lin / kXcds;
    item = idx / per;
    h = lin % kXcds + kXcds * (idx % per);
  } else {
    item = lin / a.num_heads;
    h = lin % a.num_heads;
  }
  // Items in work_order (longest first shortens the launch's tail), else
  // sequence by sequence with a sequence's later query tiles, which see
  // more keys, first.
  const int code = a.work_order != nullptr
                       ? min(max(a.work_order[item], 0), nitems - 1)
                       : item + (ntiles - 1) - 2 * (item % ntiles);
  const int s = code / ntiles;
  const int qt = code % ntiles;
  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  int q0 = a.query_start[s];
  int n = a.query_start[s + 1] - q0;
  q0 = q0 < 0 ? 0 : q0;
  n = n < 0 ? 0 : n;
  n = min(min(n, ctx), a.max_query_len);
  n = min(n, a.total_queries - q0);
  if (qt * kBM >= n) return;  // uniform over the workgroup

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;        // which 8-element half of a k-step this lane holds
  const int col = lane & 31;         // query column (B operand / accumulator column)
  const int first = ctx - n;         // position of the sequence's first query
  const int my_q = qt * kBM + wave * kQW + col;
  const bool q_ok = my_q < n;
  const int my_pos = first + my_q;   // the query's position: it sees keys 0 .. my_pos
  const int wg_last = first + min(n, (qt + 1) * kBM) - 1;   // last position in the workgroup
  const int wave_first = first + qt * kBM + wave * kQW;     // first position of the wavefront
  const int wave_last = first + min(n, qt * kBM + (wave + 1) * kQW) - 1;
  // A wavefront past the tile's last query (short query runs) still loads
  // and stages its share of every K/V tile, but computes nothing, leaving
  // its SIMD to the wavefronts of other workgroups.
  const bool wave_live = qt * kBM + wave * kQW < n;

  const int64_t head_bytes = static_cast<int64_t>(h) * D * T::kBytes;
  const uint32_t row_bytes = static_cast<uint32_t>(a.num_heads) * D * T::kBytes;
  const int64_t frame_bytes = static_cast<int64_t>(row_bytes) * a.block_size;
  const int32_t* table_row = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;
  const uint32_t max_frame = static_cast<uint32_t>(a.num_blocks - 1);

  // Q^T as the B operand: lane holds query `col`, head-dim elements
  // 16 * step + 8 * half + [0, 8).
  vec qb[kSteps];
  {
    const char* qrow = static_cast<const char*>(a.q) +
                       ((static_cast<int64_t>(q0) + my_q) * a.num_heads + h) * D * T::kBytes;
    // scale * (q . k) = |scale| * ((-q) . k) for scale < 0; flipping the
    // sign bit of every 16-bit element negates q exactly
    const uint32_t sign = a.negate_q ? 0x80008000u : 0u;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (q_ok) v = load16(qrow + (16 * st + 8 * half) * T::kBytes);
      v = u32x4{v.x ^ sign, v.y ^ sign, v.z ^ sign, v.w ^ sign};
      qb[st] = M::from_bits(v);
    }
  }

  __shared__ __attribute__((aligned(16))) uint16_t lds_kb[2][kBN][D + kPadK];
  __shared__ __attribute__((aligned(16))) uint16_t lds_vb[2][kBN][D + kPadV];
  // For block sizes whose frames a wavefront's load can cross (not a power
  // of two, or under kWaveKeys tokens): the workgroup's slice of the block
  // table (frames of keys 0 .. wg_last), clamped into the pool, read once so
  // that a tile's K/V loads need no dependent table read. Longer contexts
  // read the table directly. Otherwise each wavefront reads its frames as
  // scalars, a tile ahead of the loads that use them (tile_frames).
  __shared__ uint32_t lds_tbl[kTableCache];
  // Set when a wavefront's accumulators ended non-finite after a pass with
  // V staged in fp16.
  __shared__ int lds_wide;
  // Block sizes that are powers of two (the common case) split a token
  // position into (block, offset) with a shift and a mask. Piece i of a
  // wavefront covers kWaveKeys consecutive keys; with power-of-two frames of
  // at least that many tokens they sit in one frame (uniform frames).
  const bool pow2_block = (a.block_size & (a.block_size - 1)) == 0;
  const int block_shift = __builtin_ctz(static_cast<unsigned>(a.block_size));
  constexpr int kWaveKeys = 64 / kPieces;
  const bool uniform_frames = pow2_block && a.block_size >= kWaveKeys;
  const int n_blk = wg_last / a.block_size + 1;
  const bool tbl_in_lds = !uniform_frames && n_blk <= kTableCache;
  if (tbl_in_lds) {
    for (int b = threadIdx.x; b < n_blk; b += kWaves * 64)
      lds_tbl[b] = min(static_cast<uint32_t>(table_row[b]), max_frame);
  }
  if (threadIdx.x == 0) lds_wide = 0;
  __syncthreads();

  f32x16 o[kDBlk];
  float m, l;

  const int n_tiles = (wg_last + kBN) / kBN;
  // Each thread moves kPer 16-byte pieces of K and of V per tile. The LDS
  // tiles are double-buffered: the next tile's pieces are fetched into
  // registers while the current tile is computed, then written to the other
  // buffer (last read one tile earlier, before the previous barrier), so one
  // barrier per tile suffices.
  constexpr int kPer = kBN * kPieces / (kWaves * 64);
  static_assert(kBN * kPieces % (kWaves * 64) == 0, "tile must split evenly over the threads");
  u32x4 pk[kPer], pv[kPer];
  // With uniform frames the frame number is the same for the whole
  // wavefront's piece. Rows past the workgroup's last key are loaded from
  // the last key's row (finite data, weight 0), which keeps that property
  // and needs no per-lane branch.
  const uint32_t lane_col = 16u * (threadIdx.x % kPieces) + static_cast<uint32_t>(head_bytes);
  // Frames of the wavefront's pieces of the tile at k0 (uniform frames
  // only), read as scalars a tile before the loads that use them.
  auto tile_frames = [&](const int k0, uint32_t (&fr)[kPer]) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int key0 = (wave * 64 + i * kWaves * 64) / kPieces;
      const int tok0 = min(k0 + key0, wg_last);
      fr[i] = min(static_cast<uint32_t>(table_row[tok0 >> block_shift]), max_frame);
    }
  };
  auto fetch = [&](const int k0, const uint32_t (&fr)[kPer]) {
    if (uniform_frames) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int key0 = (wave * 64 + i * kWaves * 64) / kPieces;  // the wavefront's first key
        const int tok = min(k0 + key0 + lane / kPieces, wg_last);
        const uint32_t f = fr[i];
        const int64_t base = static_cast<int64_t>(f) * frame_bytes;
        const uint32_t off = static_cast<uint32_t>(tok & (a.block_size - 1)) * row_bytes + lane_col;
        pk[i] = load16(static_cast<const char*>(a.k_cache) + base + off);
        pv[i] = load16(static_cast<const char*>(a.v_cache) + base + off);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int piece = threadIdx.x + i * kWaves * 64;
      const int tok = k0 + piece / kPieces;
      const int c = piece % kPieces;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (tok <= wg_last) {
        int blk, inb;
        if (pow2_block) {
          blk = tok >> block_shift;
          inb = tok & (a.block_size - 1);
        } else {
          blk = tok / a.block_size;
          inb = tok - blk * a.block_size;
        }
        const uint32_t f = tbl_in_lds ? lds_tbl[blk]
                                      : min(static_cast<uint32_t>(table_row[blk]), max_frame);
        // offset inside the frame fits 32 bits (frames are under 2^31 bytes)
        const uint32_t in_frame = static_cast<uint32_t>(inb) * row_bytes +
                                  static_cast<uint32_t>(head_bytes) + 16u * c;
        const int64_t off = static_cast<int64_t>(f) * frame_bytes + in_frame;
        kv = load16(static_cast<const char*>(a.k_cache) + off);
        vv = load16(static_cast<const char*>(a.v_cache) + off);
      }
      pk[i] = kv;
      pv[i] = vv;
    }
  };
  // Write the fetched pieces to LDS buffer `buf`. With kV16 (bf16 caches),
  // V is written in fp16, rounded to nearest: a bf16 value of magnitude in
  // [2^-14, 2^16) is exactly an fp16 value (the largest bf16 value under
  // 2^16 is 65,280); 2^16 and above become infinities (a bf16 value that
  // large is at least 65,536), infinities and NaNs stay what they are.
  auto stage = [&](const int buf, auto v16) {
    constexpr bool kV16 = decltype(v16)::value;
    auto& lds_k = lds_kb[buf];
    auto& lds_v = lds_vb[buf];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int piece = threadIdx.x + i * kWaves * 64;
      const int key = piece / kPieces;
      const int c = piece % kPieces;
      *reinterpret_cast<u32x4*>(&lds_k[key][8 * c]) = pk[i];
      u32x4 vw = pv[i];
      if constexpr (kV16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t d = pv[i][w];
          const f32x2 f = {__uint_as_float(d << 16), __uint_as_float(d & 0xffff0000u)};
          vw[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
        }
      }
      *reinterpret_cast<u32x4*>(&lds_v[key][8 * c]) = vw;
    }
  };
  // Score rows in a permuted key order: row i = 8 u + 4 v + e (u < 4, v < 2,
  // e < 4) holds key 16 (u / 2) + 8 v + 4 (u % 2) + e. The accumulator gives
  // lane (query, half) rows 8 u + 4 half + e as elements e + 4 u, so its
  // elements 8 j .. 8 j + 7 are keys 16 j + 8 half + [0, 8): the layout the
  // weighted sum's B operand needs, with no exchange between lanes.
  const int krow = 16 * (col / 16) + 8 * ((col / 4) % 2) + 4 * ((col / 8) % 2) + col % 4;

  // One pass over the key tiles. kV16 (bf16 caches only): V staged in fp16
  // and the weighted sum on fp16 operands; otherwise the cache dtype's.
  auto pass = [&](auto v16) {
    constexpr bool kV16 = decltype(v16)::value;
    // bf16 weights as a high part and a residual (see below)
    constexpr bool kSplitP = kBf16 && !kV16;
    using PM = typename std::conditional<kV16, Mfma<F16>, M>::type;
    using pvec = typename PM::vec;
#pragma unroll
    for (int b = 0; b < kDBlk; ++b)
#pragma unroll
      for (int t = 0; t < 16; ++t) o[b][t] = 0.f;
    m = kNegBig;
    l = 0.f;
    uint32_t fr[kPer] = {};
    if (uniform_frames) tile_frames(0, fr);
    fetch(0, fr);
    if (uniform_frames && n_tiles > 1) tile_frames(kBN, fr);
    stage(0, v16);
    __syncthreads();
    for (int kt = 0; kt < n_tiles; ++kt) {
      const int k0 = kt * kBN;
      if (kt + 1 < n_tiles) fetch(k0 + kBN, fr);
      if (uniform_frames && kt + 2 < n_tiles) tile_frames(k0 + 2 * kBN, fr);
      auto& lds_k = lds_kb[kt & 1];
      auto& lds_v = lds_vb[kt & 1];

      if (wave_live && k0 <= wave_last) {  // the tile holds keys some query of this wavefront sees
        // S^T = K Q^T: rows = keys of the tile, columns = this wavefront's queries
        f32x16 st;
#pragma unroll
        for (int t = 0; t < 16; ++t) st[t] = 0.f;
#pragma unroll
        for (int step = 0; step < kSteps; ++step) {
          const u32x4 kbits = *reinterpret_cast<const u32x4*>(&lds_k[krow][16 * step + 8 * half]);
          st = M::run(M::from_bits(kbits), qb[step], st);
        }
        // causal mask + online softmax for the lane's query
        const bool full = k0 + kBN - 1 <= wave_first;  // every key visible to every query
        float x[16];
        float tmax = -__builtin_inff();
        if (full) {  // wavefront-uniform: no mask
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            x[t] = st[t];
            tmax = fmaxf(tmax, x[t]);
          }
        } else {
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int key = k0 + 16 * (t / 8) + 8 * half + t % 8;
            x[t] = (q_ok && key <= my_pos) ? st[t] : -__builtin_inff();
            tmax = fmaxf(tmax, x[t]);
          }
        }
        // raw scores so far; the scale (>= 0, so order-preserving) is applied
        // to the maximum here and folded into the exponent's fma below
        tmax = max_halves(tmax) * a.scale_log2;
        // Lazy rescaling: the reference maximum m moves (and O, l are
        // rescaled) only when a query's maximum grows by more than kLazy
        // (log2 units); otherwise weights are taken against the stale m and
        // stay below 2^kLazy. The common factor 2^-m cancels in O / l, so the
        // result is the same softmax; the O rescale, a multiply of every
        // accumulator, becomes rare.
        const bool grow = tmax > m + kLazy;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wavefront-uniform branch
          const float m_new = grow ? tmax : m;
          const float alpha = fast_exp2(m - m_new);
          l *= alpha;
#pragma unroll
          for (int b = 0; b < kDBlk; ++b)
#pragma unroll
            for (int t = 0; t < 16; ++t) o[b][t] *= alpha;
          m = m_new;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) x[t] = fast_exp2(__builtin_fmaf(x[t], a.scale_log2, -m));
        // With a positive scale a masked key's exponent is -inf, so its weight
        // is already exactly 0; only a zero scale (-inf * 0 = NaN) needs the
        // mask again (scale_log2 is uniform, so is the branch).
        if (!full && a.scale_log2 == 0.f) {
          // masked keys weigh exactly 0
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int key = k0 + 16 * (t / 8) + 8 * half + t % 8;
            x[t] = (q_ok && key <= my_pos) ? x[t] : 0.f;
          }
        }

        // x[8j .. 8j+7] are the weights of keys 16j + 8*half + [0, 8): already
        // the B-operand layout of the weighted sum's k-step j (see krow).
        // fp16 operands (fp16 caches, or bf16 V staged in fp16) keep 11
        // significant bits of each weight: one rounding, one MFMA, and l sums
        // the rounded weights, so that O / l is a convex combination of the
        // values with exactly the weights the matrix cores applied. The bf16
        // split keeps ~16: P = hi + lo per pair of weights, hi rounded to bf16
        // and lo the rounded residual (x - hi is exact in fp32), two MFMAs.
        pvec p_hi[2], p_lo[2];
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const f32x2 xv = {x[8 * j + e], x[8 * j + e + 1]};
            const auto hp = __builtin_convertvector(xv, typename PM::pair);
            p_hi[j][e] = hp.x;
            p_hi[j][e + 1] = hp.y;
            if constexpr (kSplitP) {
              const f32x2 hw = __builtin_convertvector(hp, f32x2);
              const auto lp =
                  __builtin_convertvector(f32x2{xv.x - hw.x, xv.y - hw.y}, typename PM::pair);
              p_lo[j][e] = lp.x;
              p_lo[j][e + 1] = lp.y;
              psum += xv.x + xv.y;
            } else {
              psum = __builtin_amdgcn_fdot2(hp, typename PM::pair{1, 1}, psum, false);
            }
          }
        l += psum;  // this lane's share; the two halves are added at the end
        // O^T += V^T P^T. The V^T operand (8 consecutive keys per lane at one
        // head-dim element) comes from the row-major V tile through
        // transposing LDS reads: in each group of 16 lanes, a 64-bit
        // transpose read hands lane l element j = (element l % 4 of the chunk
        // lane 4j + l/4 points at), so lane c points at V[kb + c/4][d0 + 4 (c %
        // 4)] and lane l receives V[kb + j][d0 + l], j = 0..3; two reads cover
        // 8 keys.
        const int grp16 = lane >> 4;
        const int c16 = lane & 15;
        auto v_operand = [&](const int b, const int j) {
          const int d0 = 32 * b + 16 * (grp16 & 1);
          const int kb = 16 * j + 8 * (grp16 >> 1);
          const v4i16 lo4 = tr_read(&lds_v[kb + (c16 >> 2)][d0 + 4 * (c16 & 3)]);
          const v4i16 hi4 = tr_read(&lds_v[kb + 4 + (c16 >> 2)][d0 + 4 * (c16 & 3)]);
          return PM::from_bits(join(lo4, hi4));
        };
        // the next V operand is read while the current one's MFMAs run; keys
        // 0-15 of the tile for every output block first, then keys 16-31
        pvec va_next = v_operand(0, 0);
#pragma unroll
        for (int n = 0; n < 2 * kDBlk; ++n) {
          const int j = n / kDBlk, b = n % kDBlk;
          const pvec va = va_next;
          if (n + 1 < 2 * kDBlk) va_next = v_operand((n + 1) % kDBlk, (n + 1) / kDBlk);
          o[b] = PM::run(va, p_hi[j], o[b]);
          if constexpr (kSplitP) o[b] = PM::run(va, p_lo[j], o[b]);
        }
      }
      if (kt + 1 < n_tiles) stage((kt + 1) & 1, v16);
      __syncthreads();
    }
  };

  if constexpr (kBf16) {
    bool split = a.split_weights != 0;
    if (!split) {
      pass(std::true_type{});
      // A V value out of fp16's range was staged as an infinity or NaN, and
      // every wavefront that read its tile (the one holding the workgroup's
      // last query reads every tile) ends with a non-finite accumulator:
      // p * inf, or 0 * inf = NaN for a key a query does not see. Then the
      // workgroup redoes all its tiles with the bf16 split (the LDS buffers
      // are no longer read, so the second pass may restage them at once),
      // through the same code as a split launch, so with the same bits.
      // (Non-finite q or k also lead here, to the same non-finite result.)
      float probe = 0.f;  // NaN iff an accumulator is infinite or NaN
#pragma unroll
      for (int b = 0; b < kDBlk; ++b)
#pragma unroll
        for (int t = 0; t < 16; ++t) probe = __builtin_fmaf(o[b][t], 0.f, probe);
      if (probe != probe) lds_wide = 1;
      __syncthreads();
      split = lds_wide != 0;
    }
    if (split) pass(std::false_type{});
  } else {
    pass(std::false_type{});
  }

  l = sum_halves(l);
  if (!q_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = (static_cast<int64_t>(q0) + my_q) * a.num_heads + h;
#pragma unroll
  for (int b = 0; b < kDBlk; ++b)
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int d = 32 * b + (t % 4) + 8 * (t / 4) + 4 * half;
      const float r = o[b][t] * inv;
      if (a.out_f32)
        static_cast<float*>(a.out)[orow * D + d] = r;
      else
        static_cast<uint16_t*>(a.out)[orow * D + d] = static_cast<uint16_t>(narrow_bits(T{}, r));
    }
}


template <typename T, int D>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  const int ntiles = (a.max_query_len + kBM - 1) / kBM;
  dim3 grid(a.num_seqs * ntiles * a.num_heads);
  return launch_timed(prefill_kernel<T, D>, grid, dim3(kWaves * 64), stream, a);
}

}  // namespace

bool prefill_supported(Dtype dt, int head_dim) {
  return (dt == Dtype::BF16 || dt == Dtype::F16) && (head_dim == 64 || head_dim == 128);
}

hipError_t launch_prefill(const PrefillArgs& a, Dtype dt, int head_dim, hipStream_t stream) {
  if (dt == Dtype::BF16) {
    if (head_dim == 64) return launch_t<BF16, 64>(a, stream);
    if (head_dim == 128) return launch_t<BF16, 128>(a, stream);
  } else if (dt == Dtype::F16) {
    if (head_dim == 64) return launch_t<F16, 64>(a, stream);
    if (head_dim == 128) return launch_t<F16, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
