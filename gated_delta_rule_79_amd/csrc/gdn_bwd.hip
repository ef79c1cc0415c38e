// Chunkwise backward of the gated delta rule (placeholder until the
// backward kernels land: reports the request as unsupported).
#include "gdn_chunk_common.hpp"

namespace gdn {

size_t bwd_workspace_bytes(const Problem& p) { (void)p; return 0; }

hipError_t launch_bwd(const Problem&, const void*, const void*, const void*,
                      const void*, const void*, const float*, const void*,
                      const float*, void*, void*, void*, float*, float*,
                      float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace gdn
