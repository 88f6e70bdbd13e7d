// Chunked causal prefill (placeholder until the MFMA kernel lands).
#include "kernels.h"

namespace gattn {
hipError_t launch_prefill(const PrefillArgs &, int, bool, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gattn
