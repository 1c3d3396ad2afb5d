// gdn_chunked.hip -- chunk-parallel prefill on MFMA (not built yet: every
// shape goes to the token-sequential kernel).
#include "gdn_launch.h"

namespace gdn {

bool chunked_supported(int, int, int, int) { return false; }

size_t chunked_workspace_bytes(int64_t, int64_t, int, int, int) { return 0; }

hipError_t launch_prefill_chunked(const PrefillArgs&, void*, size_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace gdn
