// Host-side launchers of the benchmark-support probes that are not part of
// the attention path (internal interface between the C ABI layer and
// stream_read.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Frame-pattern read: see pa_frame_read in include/paged_attn.h.
hipError_t launch_frame_read(const void* buf, const int32_t* frame_order, int64_t num_frames,
                             int64_t frame_bytes, int32_t groups, int64_t group_stride,
                             int32_t pieces, int64_t piece_stride, int32_t piece_bytes,
                             int32_t frames_per_unit, uint32_t* sink, hipStream_t stream);

}  // namespace pa
