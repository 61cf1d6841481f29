// Host-side helpers shared by the C-ABI translation units (no HIP types).
#pragma once

#include "muse_attn.h"

namespace muse {

// Record a formatted message for muse_last_error() and return `s`.
muse_status set_error(muse_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
const char *last_error();

}  // namespace muse
