// k_chunk.hip -- chunked (WY / UT-transform) prefill form of the recurrence.
#include <hip/hip_runtime.h>

#include "gdn.h"
#include "launch.hpp"

namespace gdn {

size_t chunked_workspace_bytes(int, int, int, int, int, int) { return 256; }

int launch_recur_chunked(const RecurArgs &, int, void *, size_t, hipStream_t) {
  return GDN_ERR_UNSUPPORTED;
}

}  // namespace gdn
