// chunk_mfma.hip -- chunk-parallel MFMA prefill (placeholder: not yet enabled).
#include "gdn_internal.h"

namespace gdn {
bool chunk_mfma_supports(const PrefillArgs &) { return false; }
size_t chunk_mfma_workspace(const PrefillArgs &) { return 0; }
hipError_t launch_chunk_mfma(const PrefillArgs &) { return hipErrorNotSupported; }
}  // namespace gdn
