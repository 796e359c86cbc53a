// Draft-head tree expansion (placeholder until the draft kernels land).
#include "draft.h"

namespace eagle {
size_t draft_workspace(const eagle_dims*, const eagle_draft_params*, int, int) { return 0; }
}  // namespace eagle

extern "C" int eagle_draft_expand(const eagle_dims*, const eagle_draft_params*, const void*, const eagle_layer_w*,
                                  const void*, const void*, const void*, int32_t, const float*, const int32_t*,
                                  const void*, const void*, const eagle_cache_layout*, const int32_t*, int32_t,
                                  int32_t*, int32_t*, int32_t*, float*, void*, size_t, eagle_timer*, int32_t*,
                                  void*) {
  return EAGLE_ERR_UNSUPPORTED;
}
