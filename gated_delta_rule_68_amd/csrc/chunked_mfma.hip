// Matrix-core (MFMA) chunked kernel: not yet instantiated in this build.
#include "gdr_internal.h"

namespace gdr {

bool chunked_mfma_supports(const Problem &) { return false; }

hipError_t launch_chunked_mfma(const Problem &, const FwdArgs &, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace gdr
