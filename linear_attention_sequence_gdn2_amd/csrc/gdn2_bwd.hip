// gdn2_bwd.hip -- backward kernels (placeholder until the reverse sweep lands).
#include "gdn2_device.h"
#include "gdn2_kernels.h"

namespace gdn2 {
hipError_t launch_bwd_reverse(const BwdArgs &, int, int, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_chunk(const BwdArgs &, int, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gdn2
