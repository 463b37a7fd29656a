// Paged decode partition pass for bf16 caches (its own file, so that the
// dtypes' instantiations compile in parallel).
#include "paged_decode.h"

namespace pa {

hipError_t decode_dispatch_bf16(const DecodeArgs& a, const GroupArgs* g, int head_dim,
                                hipStream_t stream) {
  return dispatch_dim<BF16>(a, g, head_dim, stream);
}

}  // namespace pa
