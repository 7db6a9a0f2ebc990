// Decode-sized (M <= 32) layer with the transform fused into the GEMM.
// Placeholder until the fused kernel lands: reports the path as unavailable.
#include "mx_common.h"

namespace macaq {

bool linear_fused_supported(int64_t, int64_t, int64_t, int64_t) { return false; }
size_t linear_fused_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }
hipError_t launch_linear_fused(const void*, bool, const float*, const uint8_t*, const uint8_t*, int64_t,
                               int64_t, int64_t, float*, void*, size_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace macaq
