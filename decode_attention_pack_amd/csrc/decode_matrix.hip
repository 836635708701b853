// decode_matrix.hip -- matrix-core (MFMA) decode attention over the KIVI cache.
// Not available yet: every shape is routed to the scalar kernel.
#include "kivi_internal.hpp"

namespace kivi {

bool decode_matrix_supported(const DecodeArgs &) { return false; }

hipError_t launch_decode_matrix(const DecodeArgs &, int64_t, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace kivi
