// Placeholder predicates: no matrix-core path is registered yet.
#include "common.hpp"

namespace ttt {
bool linear_mfma_supported(const LinearArgs&, bool) { return false; }
hipError_t launch_linear_mfma(const LinearArgs&, hipStream_t) { return hipErrorNotSupported; }
bool delta_fast_supported(const LinearArgs&, bool) { return false; }
hipError_t launch_delta_fast(const LinearArgs&, bool, hipStream_t) { return hipErrorNotSupported; }
bool mlp_fast_supported(const MlpArgs&, bool) { return false; }
hipError_t launch_mlp_fast(const MlpArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ttt
