// Launchers of kernels that are not built yet: they refuse the call.
#include "internal.hpp"

namespace kvf8 {

void decode_plan(int32_t, int32_t, int32_t, int32_t, int32_t, int32_t *splits, int32_t *chunk_tokens) {
    *splits = 1;
    *chunk_tokens = 0;
}
hipError_t launch_decode(const DecodeArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_kshift(const KShiftArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kvf8
