// Launchers of kernels that are not built yet: they refuse the call.
#include "internal.hpp"

namespace kvf8 {

hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kvf8
