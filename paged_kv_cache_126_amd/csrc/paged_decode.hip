// Paged decode attention for gfx950: a partition pass and a log-sum-exp merge.
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
// Work decomposition. One workgroup per (head, context partition, sequence),
// head fastest so the workgroups in flight together read whole frames (all
// heads of a token are adjacent). The workgroup's kNW wavefronts take the
// partition's chunks of kCH tokens round robin. Inside a wavefront, each
// cache row (one token's D elements of head h) is spread over kLPR lanes
// holding 16 bytes each, so one load instruction moves kRPL whole rows and
// every lane issues 16-byte loads. q . k is a per-lane dot product (packed
// dot2 instructions for 16-bit types) finished by DPP sums inside each group
// of kLPR lanes. Softmax is online: each lane group keeps its own running
// maximum m (in log2 units), sum l and fp32 accumulator for its kVEC output
// elements; groups are combined by cross-lane shuffles, wavefronts through
// LDS, both with the log-sum-exp rule. The context partitions of one
// sequence are combined the same way by the merge kernel.
//
// Masking: tokens at or past ctx are never loaded; their score is -inf and
// their weight exactly 0, so NaN-filled unused slots cannot leak in. The
// running maximum starts at a large finite negative value so that no
// inf - inf ever reaches exp2.
#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr float kNegBig = -1.0e30f;
constexpr int kNW = 8;  // wavefronts per workgroup
constexpr int kU = 4;   // row loads per lane per chunk (for each of K and V)

template <bool kStream>
__device__ __forceinline__ u32x4 load_row(const char* p) {
  if constexpr (kStream)
    return load16_stream(p);
  else
    return load16(p);
}

template <typename T, int D>
struct Tiling {
  static constexpr int kVEC = Vec<T>::kElems;  // elements a lane holds per row
  static constexpr int kLPR = D / kVEC;        // lanes per cache row
  static constexpr int kRPL = 64 / kLPR;       // rows per wavefront load
  static constexpr int kCH = kU * kRPL;        // tokens per chunk
  static_assert(kLPR >= 1 && kLPR <= 64 && (64 % kLPR) == 0, "row must tile a wavefront");
};

// kStream selects non-temporal K/V loads (frames read once) or ordinary
// cached loads (frames shared by several sequences of the call).
template <typename T, int D, int BT, bool kStream>
__global__ __launch_bounds__(kNW * 64) void decode_partition_kernel(DecodeArgs a) {
  using Tl = Tiling<T, D>;
  constexpr int VEC = Tl::kVEC, LPR = Tl::kLPR, RPL = Tl::kRPL, CH = Tl::kCH;
  // Uniform translation: with a compile-time block size that is a multiple
  // of the rows per load, the kRPL rows of one load share a frame, so the
  // frame is read once per load as a scalar.
  constexpr bool kUniformFrame = BT > 0 && (BT % RPL) == 0;

  const int h = blockIdx.x;
  const int part = blockIdx.y;
  const int s = blockIdx.z;
  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int n_parts = ctx <= a.part_tokens ? 1 : (ctx + a.part_tokens - 1) / a.part_tokens;
  if (part >= n_parts) return;  // uniform over the workgroup
  const int tok_begin = part * a.part_tokens;
  const int tok_end = min(ctx, tok_begin + a.part_tokens);

  // readfirstlane tells the compiler the wavefront index is uniform, so the
  // chunk loop, block-table reads and frame arithmetic stay scalar.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int grp = lane / LPR;  // which of the kRPL rows of a load this lane holds
  const int col = lane % LPR;  // which 16-byte piece of that row

  const int32_t* table_row = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;
  // Byte strides of the [NB, B, H, D] caches: one token row (all heads) and
  // one frame. The host guarantees frame_bytes < 2^31, so offsets inside a
  // frame fit 32 bits; frame bases are 64-bit scalars.
  const uint32_t row_bytes = static_cast<uint32_t>(a.num_heads) * D * T::kBytes;
  const int64_t frame_bytes = static_cast<int64_t>(row_bytes) * a.block_size;
  const uint32_t lane_bytes = (static_cast<uint32_t>(h) * D + col * VEC) * T::kBytes;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  const uint32_t max_frame = static_cast<uint32_t>(a.num_blocks - 1);  // num_blocks <= 2^31

  const u32x4 qv = load16(static_cast<const char*>(a.q) +
                          ((static_cast<int64_t>(s) * a.num_heads + h) * D + col * VEC) * T::kBytes);

  float m = kNegBig;
  float l = 0.f;
  float acc[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc[j] = 0.f;

  // One chunk: kU row loads of K and of V per lane, then the online-softmax
  // update. kMasked is false for chunks wholly inside the context, which
  // then load without any per-lane condition.
  auto attend_chunk = [&](const int t0, auto masked) {
    constexpr bool kMasked = decltype(masked)::value;
    u32x4 kv[kU], vv[kU];
    bool valid[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) valid[u] = !kMasked || (t0 + u * RPL + grp < tok_end);
    if constexpr (kUniformFrame) {
      // All block-table reads of the chunk first (scalar loads). A load
      // wholly past ctx reads the last valid table entry instead (its rows
      // are masked), so table columns past ceil(ctx / B) are never read.
      uint32_t frame[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t tu = static_cast<uint32_t>(t0 + u * RPL);  // wave-uniform
        const uint32_t tc = kMasked ? min(tu, static_cast<uint32_t>(tok_end - 1)) : tu;
        frame[u] = static_cast<uint32_t>(table_row[tc / BT]);
      }
      int64_t step_base[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t tu = static_cast<uint32_t>(t0 + u * RPL);
        // Out-of-range (or negative) entries are clamped into the pool.
        const uint32_t f = min(frame[u], max_frame);
        step_base[u] = static_cast<int64_t>(f) * frame_bytes + static_cast<int64_t>(tu % BT) * row_bytes;
      }
      const uint32_t lane_off = grp * row_bytes + lane_bytes;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        u32x4 kz = {0u, 0u, 0u, 0u}, vz = {0u, 0u, 0u, 0u};
        if (valid[u]) {
          kz = load_row<kStream>(kbase + step_base[u] + lane_off);
          vz = load_row<kStream>(vbase + step_base[u] + lane_off);
        }
        kv[u] = kz;
        vv[u] = vz;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        u32x4 kz = {0u, 0u, 0u, 0u}, vz = {0u, 0u, 0u, 0u};
        if (valid[u]) {
          const int64_t off =
              token_row(table_row, t0 + u * RPL + grp, a.block_size, a.num_blocks) * row_bytes +
              lane_bytes;
          kz = load_row<kStream>(kbase + off);
          vz = load_row<kStream>(vbase + off);
        }
        kv[u] = kz;
        vv[u] = vz;
      }
    }

    float sc[kU];
    float cmax = kNegBig;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float d = group_sum<LPR>(dot16(T{}, qv, kv[u]));
      sc[u] = valid[u] ? d * a.scale_log2 : -__builtin_inff();
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
  };

  const int n_chunks = (tok_end - tok_begin + CH - 1) / CH;
  for (int chunk = wave; chunk < n_chunks; chunk += kNW) {
    const int t0 = tok_begin + chunk * CH;
    if (t0 + CH <= tok_end)
      attend_chunk(t0, std::false_type{});
    else
      attend_chunk(t0, std::true_type{});
  }

  // Combine the kRPL lane groups of the wavefront (lanes col, col + LPR, ...).
#pragma unroll
  for (int x = LPR; x < 64; x <<= 1) {
    const float m_o = __shfl_xor(m, x);
    const float l_o = __shfl_xor(l, x);
    const float m_n = fmaxf(m, m_o);
    const float fa = fast_exp2(m - m_n);
    const float fb = fast_exp2(m_o - m_n);
    l = l * fa + l_o * fb;
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] = acc[j] * fa + __shfl_xor(acc[j], x) * fb;
    m = m_n;
  }

  // Combine the wavefronts through LDS.
  __shared__ float s_m[kNW];
  __shared__ float s_l[kNW];
  __shared__ float s_acc[kNW][D];
  if (grp == 0) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) s_acc[wave][col * VEC + j] = acc[j];
    if (col == 0) {
      s_m[wave] = m;
      s_l[wave] = l;
    }
  }
  __syncthreads();

  float M = kNegBig;
#pragma unroll
  for (int w = 0; w < kNW; ++w) M = fmaxf(M, s_m[w]);
  float fw[kNW];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    fw[w] = fast_exp2(s_m[w] - M);
    L += s_l[w] * fw[w];
  }
  const int64_t sh = static_cast<int64_t>(s) * a.num_heads + h;
  for (int e = threadIdx.x; e < D; e += kNW * 64) {
    float O = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) O += s_acc[w][e] * fw[w];
    if (n_parts == 1) {
      const float r = L > 0.f ? O / L : 0.f;
      const int64_t o = sh * D + e;
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
      a.ws_acc[p * D + e] = O;
      if (e == 0) {
        a.ws_ml[2 * p] = M;
        a.ws_ml[2 * p + 1] = L;
      }
    }
  }
}

// Log-sum-exp merge of a sequence's partitions: with M = max_p m_p,
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  int n_parts = ctx <= a.part_tokens ? 1 : (ctx + a.part_tokens - 1) / a.part_tokens;
  if (n_parts <= 1) return;  // written by the partition pass
  n_parts = min(n_parts, a.max_parts);
  const int64_t sh = static_cast<int64_t>(s) * a.num_heads + h;
  const float* ml = a.ws_ml + 2 * sh * a.max_parts;
  const float* pacc = a.ws_acc + sh * a.max_parts * D;
  float M = kNegBig;
  for (int p = 0; p < n_parts; ++p) M = fmaxf(M, ml[2 * p]);
  for (int e = threadIdx.x; e < D; e += blockDim.x) {
    float L = 0.f, O = 0.f;
    for (int p = 0; p < n_parts; ++p) {
      const float f = fast_exp2(ml[2 * p] - M);
      L += ml[2 * p + 1] * f;
      O += pacc[static_cast<int64_t>(p) * D + e] * f;
    }
    const float r = L > 0.f ? O / L : 0.f;
    const int64_t o = sh * D + e;
    if constexpr (T::kBytes == 4) {
      static_cast<float*>(a.out)[o] = r;
    } else {
      if (a.out_f32)
        static_cast<float*>(a.out)[o] = r;
      else
        static_cast<uint16_t*>(a.out)[o] = static_cast<uint16_t>(narrow_bits(T{}, r));
    }
  }
}

template <typename T, int D, int BT>
hipError_t launch_part(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.num_heads, a.max_parts, a.num_seqs);
  if (a.stream_loads)
    return launch_timed(decode_partition_kernel<T, D, BT, true>, grid, dim3(kNW * 64), stream, a);
  return launch_timed(decode_partition_kernel<T, D, BT, false>, grid, dim3(kNW * 64), stream, a);
}

// Block sizes with a uniform-frame specialisation; other sizes take the
// per-lane translation path (BT = 0).
template <typename T, int D>
hipError_t dispatch_block(const DecodeArgs& a, hipStream_t stream) {
  constexpr int RPL = Tiling<T, D>::kRPL;
  switch (a.block_size) {
    case 8:
      if constexpr (8 % RPL == 0) return launch_part<T, D, 8>(a, stream);
      break;
    case 16:
      if constexpr (16 % RPL == 0) return launch_part<T, D, 16>(a, stream);
      break;
    case 32:
      if constexpr (32 % RPL == 0) return launch_part<T, D, 32>(a, stream);
      break;
    case 64:
      if constexpr (64 % RPL == 0) return launch_part<T, D, 64>(a, stream);
      break;
    default:
      break;
  }
  return launch_part<T, D, 0>(a, stream);
}

template <typename T>
hipError_t dispatch_dim(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 16: return dispatch_block<T, 16>(a, stream);
    case 32: return dispatch_block<T, 32>(a, stream);
    case 64: return dispatch_block<T, 64>(a, stream);
    case 128: return dispatch_block<T, 128>(a, stream);
    case 256: return dispatch_block<T, 256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
hipError_t launch_merge_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.num_heads, a.num_seqs);
  const int threads = D < 64 ? 64 : (D > 256 ? 256 : D);
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), grid, dim3(threads), 0, stream, a);
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

int chunk_tokens(Dtype dt, int head_dim) {
  const int bytes = dt == Dtype::F32 ? 4 : 2;
  if (head_dim <= 0 || (head_dim * bytes) % 16 != 0) return 0;
  const int lpr = head_dim * bytes / 16;
  if (lpr > 64 || 64 % lpr != 0) return 0;
  return kU * (64 / lpr);
}

hipError_t launch_decode_partitions(const DecodeArgs& a, Dtype dt, int head_dim,
                                    hipStream_t stream) {
  switch (dt) {
    case Dtype::F32: return dispatch_dim<F32>(a, head_dim, stream);
    case Dtype::F16: return dispatch_dim<F16>(a, head_dim, stream);
    case Dtype::BF16: return dispatch_dim<BF16>(a, head_dim, stream);
  }
  return hipErrorInvalidValue;
}

// The merge kernel only needs the output type: the cache dtype matters for
// the narrowing of a 16-bit output.
hipError_t launch_decode_merge(const DecodeArgs& a, Dtype dt, int head_dim, hipStream_t stream) {
  switch (dt) {
    case Dtype::F32: return merge_dim<F32>(a, head_dim, stream);
    case Dtype::F16: return merge_dim<F16>(a, head_dim, stream);
    case Dtype::BF16: return merge_dim<BF16>(a, head_dim, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
