// Backward kernels of the CARVE key-axis gated delta rule on gfx950 (in progress).
#include "carve_device.h"
#include "carve_internal.h"

namespace carve {

hipError_t launch_bwd_state(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_chunk(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace carve
