// Launch stubs for a host-only build of the library's C ABI (csrc/gattn.cpp), used by the CPU
// sanitizer tests: argument validation, split planning and workspace sizing run for real under
// AddressSanitizer and UndefinedBehaviorSanitizer, while every kernel launch and graph capture fails with
// hipErrorInvalidValue (reported as GATTN_ERR_HIP), so a library linked with them never computes a result.
#include "kernels.h"

namespace gattn {

hipError_t launch_kv_append(const AppendArgs &, int, int, bool, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_decode_split(const DecodeArgs &, int, bool, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_decode_split_fp8(const DecodeArgs &, int, bool, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_combine(int, int, int, int, const float *, const float *, uint16_t *, float *, hipStream_t,
                          const CombineRows &) {
    return hipErrorInvalidValue;
}
hipError_t launch_prefill(const PrefillArgs &, int, bool, int, hipStream_t) { return hipErrorInvalidValue; }
bool decode_merges_slots(int, bool, int, int64_t) { return false; }
hipError_t noalloc_scratch(void **, size_t *) { return hipErrorInvalidValue; }
hipError_t graph_capture_begin(hipStream_t *s) {
    *s = nullptr;
    return hipErrorInvalidValue;
}
hipError_t graph_capture_end(hipStream_t, void **exec) {
    *exec = nullptr;
    return hipErrorInvalidValue;
}
hipError_t graph_launch(void *, hipStream_t) { return hipErrorInvalidValue; }
void graph_free(void *) {}

}  // namespace gattn
