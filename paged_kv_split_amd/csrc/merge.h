// Internal interface between the C-ABI host layer (pdattn.hip) and the
// partial-state merge kernel (merge.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdattn {

struct MergeStatesParams {
  const float* partial_out;  // [S][R][D]
  const float* partial_lse;  // [S][R], natural log
  float* out;                // [R][D]
  float* lse;                // [R] or null
  int64_t num_rows;          // R
  int32_t num_partials;      // S
};

hipError_t launch_merge_states(const MergeStatesParams& p, int head_dim, hipStream_t stream);

}  // namespace pdattn
