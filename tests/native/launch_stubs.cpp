// Test-only stand-ins for the kernel launchers, so that the host code of the store, the planner
// and the C ABI can be built and fuzzed under the address and undefined-behaviour sanitizers
// without a GPU. The fuzzer uses metadata-only stores, on which no device call is reached; a
// launcher called anyway reports an error.
#include "launch.h"

namespace piclink {

hipError_t launch_store_fill(const LayerShape &, void *, void *, const void *, const void *, const FillPages &,
                             hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_scatter(const LayerShape &, void *, void *, const void *, const void *, const float *,
                          const ScatterDesc *, int, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_prepare(const LayerShape &, void *, void *, const void *, const void *, const float *,
                          const PageDesc *, const int32_t *, int, const ScatterDesc *, int, void *, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_attention(const LayerShape &, const void *, const void *, const void *, const float *,
                            const AttnTables &, void *, float *, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_merge(const LayerShape &, const AttnTables &, void *, float *, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t static_scratch(void **) { return hipErrorNotSupported; }
hipError_t launch_decode(const LayerShape &, const void *, const void *, const void *, void *, void *, const float *,
                         const DecodeTables &, void *, float *, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace piclink
