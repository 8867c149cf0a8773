// api_internal.h -- pieces of the C ABI's implementation (api.cpp) shared with entry
// points defined next to device code.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/hypic.h"

namespace hypic {

// records `msg` as the calling thread's last error and returns `st`
hypic_status api_error(hypic_status st, const char* msg);

// hypic_seam_advance with the workspace already chosen: every argument check (the
// workspace's size and alignment included), then the launches on `stream`.
hypic_status seam_advance_with(const hypic_dims* dims, int32_t n_chain, int32_t n_step, int32_t w,
                               const int64_t* seam_start, int64_t n_tokens, const void* q, const void* k,
                               const void* v, const void* g, const void* beta, float scale,
                               const int32_t* pair_id, int32_t n_pair, const void* T_cache,
                               const float* S_cache, float* S_run, float* out, void* workspace,
                               size_t workspace_bytes, void* stream);

}  // namespace hypic
