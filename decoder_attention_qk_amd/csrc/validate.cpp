// Pure host checks (no HIP): the packed-layout validator and the error slot.
// Model page, _validate_thd_documents: packed document lengths are checked and
// the real maximum length is what sizes the work.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "muse_attn.h"
#include "host_util.hpp"

namespace muse {

static thread_local std::string g_last_error;

muse_status set_error(muse_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

void clear_error() { g_last_error.clear(); }

const char *last_error() { return g_last_error.c_str(); }

}  // namespace muse

extern "C" muse_status muse_validate_cu_seqlens(const int32_t *cu, int32_t num_segments,
                                                int32_t total_tokens, int32_t max_seqlen) {
  using muse::set_error;
  if (!cu) return set_error(MUSE_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if (num_segments < 1) return set_error(MUSE_ERR_INVALID_ARG, "num_segments %d < 1", num_segments);
  if (cu[0] != 0) return set_error(MUSE_ERR_INVALID_ARG, "cu_seqlens[0] = %d, expected 0", cu[0]);
  for (int32_t i = 0; i < num_segments; ++i) {
    const int64_t len = (int64_t)cu[i + 1] - cu[i];
    if (len < 0)
      return set_error(MUSE_ERR_INVALID_ARG, "cu_seqlens decreases at %d (%d -> %d)", i, cu[i], cu[i + 1]);
    if (len > max_seqlen)
      return set_error(MUSE_ERR_INVALID_ARG, "segment %d has length %lld > max_seqlen %d", i,
                       (long long)len, max_seqlen);
  }
  if (cu[num_segments] != total_tokens)
    return set_error(MUSE_ERR_INVALID_ARG, "cu_seqlens[%d] = %d, expected total_tokens %d", num_segments,
                     cu[num_segments], total_tokens);
  muse::clear_error();
  return MUSE_OK;
}

extern "C" const char *muse_status_string(muse_status s) {
  switch (s) {
    case MUSE_OK: return "MUSE_OK";
    case MUSE_ERR_INVALID_ARG: return "MUSE_ERR_INVALID_ARG";
    case MUSE_ERR_UNSUPPORTED: return "MUSE_ERR_UNSUPPORTED";
    case MUSE_ERR_DEVICE: return "MUSE_ERR_DEVICE";
  }
  return "MUSE_ERR_UNKNOWN";
}

extern "C" const char *muse_last_error(void) { return muse::last_error(); }

extern "C" const char *muse_version(void) { return "0.1.0"; }
