// Chunked-prefill attention (placeholder until the MFMA kernel lands).
#include "pa_internal.h"

namespace pa {

int prefill_tile_rows(int head_dim) { return head_dim == 64 ? 128 : 128; }

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int group, hipStream_t s) {
  (void)a; (void)head_dim; (void)group; (void)s;
  return hipErrorNotSupported;
}

}  // namespace pa
