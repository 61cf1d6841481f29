// Opt-in checks of the device-side layout arrays (MUSE_DEBUG_VALIDATE=1):
// the arrays are copied to the host in the caller's stream order, which
// synchronises that stream -- the only place the library waits.  Model page,
// _validate_thd_documents (packed boundaries) and MuseSparkTextModel.forward
// (local position_ids, which index the RoPE table).
#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <vector>

#include "host_util.hpp"

namespace muse {

bool debug_validate_enabled() {
  const char *e = std::getenv("MUSE_DEBUG_VALIDATE");
  return e && e[0] == '1';
}

static bool copy_to_host(void *dst, const void *src, size_t bytes, void *stream) {
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, (hipStream_t)stream) == hipSuccess &&
         hipStreamSynchronize((hipStream_t)stream) == hipSuccess;
}

muse_status debug_check_cu_seqlens(const muse_layout *l, void *stream) {
  if (l->num_segments >= (1 << 26)) return MUSE_OK;
  std::vector<int32_t> host((size_t)l->num_segments + 1);
  if (!copy_to_host(host.data(), l->cu_seqlens, host.size() * sizeof(int32_t), stream))
    return set_error(MUSE_ERR_DEVICE, "copying cu_seqlens for validation failed");
  return muse_validate_cu_seqlens(host.data(), l->num_segments, l->total_tokens, l->max_seqlen);
}

muse_status debug_check_positions(const int32_t *position_ids, int64_t n_tokens, int32_t n_pos, void *stream) {
  if (!position_ids || n_tokens <= 0) return MUSE_OK;
  std::vector<int32_t> host((size_t)n_tokens);
  if (!copy_to_host(host.data(), position_ids, host.size() * sizeof(int32_t), stream))
    return set_error(MUSE_ERR_DEVICE, "copying position_ids for validation failed");
  for (int64_t t = 0; t < n_tokens; ++t)
    if (host[(size_t)t] < 0 || host[(size_t)t] >= n_pos)
      return set_error(MUSE_ERR_INVALID_ARG, "position_ids[%lld] = %d is outside the table's [0, %d)",
                       (long long)t, host[(size_t)t], n_pos);
  return MUSE_OK;
}

}  // namespace muse
