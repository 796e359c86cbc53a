// Internal interface of the draft-head tree expansion.
#pragma once

#include "common.h"

namespace eagle {

size_t draft_workspace(const eagle_dims* d, const eagle_draft_params* p, int batch, int max_prefix);
int launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// Workspace of eagle_draft_kv_commit (decode.hip); 0 for unsupported arguments.
size_t draft_kv_workspace(const eagle_dims* d, int batch, int max_accept);

}  // namespace eagle
