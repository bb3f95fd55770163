// Outer-loop backward -- not built yet.
#include "ttt_device.hpp"

namespace ttt {
size_t bwd_generic_lds_bytes(int, int, int, int) { return 0; }
size_t bwd_work_floats_per_head(int, int, int, int) { return 0; }
hipError_t launch_bwd_generic(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_finalize(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ttt
