// Paged decode attention: host entry points of the partition pass (one file
// per cache dtype compiles its launches) and the log-sum-exp merge. The
// kernels and what they compute are described in paged_decode.h.
#include "paged_decode.h"

namespace pa {

int chunk_tokens(Dtype dt, int head_dim, int num_heads) {
  const int bytes = dt == Dtype::F32 ? 4 : 2;
  if (head_dim <= 0 || num_heads <= 0 || (head_dim * bytes) % 16 != 0) return 0;
  const int lpr = head_dim * bytes / 16;
  if (lpr > 64 || 64 % lpr != 0) return 0;
  return kU * (64 / lpr) / heads_per_group(head_dim * bytes, num_heads);
}

int heads_per_workgroup(Dtype dt, int head_dim, int num_heads) {
  if (chunk_tokens(dt, head_dim, num_heads) <= 0) return 0;
  return heads_per_group(head_dim * (dt == Dtype::F32 ? 4 : 2), num_heads);
}

hipError_t launch_decode_partitions(const DecodeArgs& a, Dtype dt, int head_dim,
                                    hipStream_t stream) {
  return launch_decode_groups(a, nullptr, dt, head_dim, stream);
}

hipError_t launch_decode_groups(const DecodeArgs& a, const GroupArgs* g, Dtype dt, int head_dim,
                                hipStream_t stream) {
  switch (dt) {
    case Dtype::F32: return decode_dispatch_f32(a, g, head_dim, stream);
    case Dtype::F16: return decode_dispatch_f16(a, g, head_dim, stream);
    case Dtype::BF16: return decode_dispatch_bf16(a, g, head_dim, stream);
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
