// Internal interface of the draft-head tree expansion.
#pragma once

#include "common.h"

namespace eagle {

size_t draft_workspace(const eagle_dims* d, const eagle_draft_params* p, int batch, int max_prefix);
int launch_fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace eagle
