// Host-side helpers shared by the C-ABI translation units (no HIP types).
#pragma once

#include "muse_attn.h"

namespace muse {

// Record a formatted message for muse_last_error() and return `s`.
muse_status set_error(muse_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
const char *last_error();

// MUSE_DEBUG_VALIDATE=1 checks of device layout arrays (debug_check.cpp):
// each copies its array to the host, synchronising `stream` (a hipStream_t).
bool debug_validate_enabled();
muse_status debug_check_cu_seqlens(const muse_layout *layout, void *stream);
muse_status debug_check_positions(const int32_t *position_ids, int64_t n_tokens, int32_t n_pos, void *stream);

}  // namespace muse
