// k_mfma.hip -- MFMA chunk path (not yet built; the token-serial path serves all calls).
#include "gtr_internal.hpp"

namespace gtr {
bool mfma_supported(const GlaArgs &) { return false; }
hipError_t mfma_summary(const GlaArgs &, float *, float *, int, int, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t mfma_output(const GlaArgs &, const float *, int, int, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace gtr
