// Predicates of the matrix-core paths that are not written yet: these shapes run on the
// generic kernels.
#include "common.hpp"

namespace ttt {
bool mlp_fast_supported(const MlpArgs&, bool) { return false; }
hipError_t launch_mlp_fast(const MlpArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ttt
