// Chunked prompt pass of libgdn (gfx950).
#include "gdn_prefill.h"

namespace gdn {

bool prefill_supported(int, int, int, int) { return false; }

size_t prefill_workspace_bytes(int, int, int, int, int, int) { return 0; }

hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gdn
