// Tuned forward scan (bf16 MFMA) -- not built yet; the portable kernel serves every config.
#include "ttt_device.hpp"

namespace ttt {
bool fwd_mfma_supported(const ScanParams&) { return false; }
hipError_t launch_fwd_mfma(const ScanParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ttt
