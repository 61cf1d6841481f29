// C ABI of libmuseattn: argument validation on the host, then kernel launches
// on the caller's stream.  No allocation (scratch memory is the caller's
// workspace), no synchronisation (the opt-in debug checks of debug_check.cpp
// aside), no state besides the per-thread error message.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "host_util.hpp"
#include "kernels.hpp"
#include "muse_attn.h"

namespace muse {
namespace {

struct Geometry {
  int64_t n_tokens;
  int d, hq, hkv, group;
  bool thd;
  int nseg;
  int maxlen;
};

struct Range {
  const void *p;
  int64_t bytes;
  const char *name;
  int align = 16;  // bytes; the kernels move bf16 and fp32 tensors in 16-byte vectors
};

bool ranges_overlap(const Range &a, const Range &b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

// Every given pointer must be aligned as its range requires, and each output
// must not overlap any input or any other output.
muse_status check_disjoint(const std::vector<Range> &inputs, const std::vector<Range> &outputs) {
  for (const auto *list : {&inputs, &outputs})
    for (const Range &r : *list)
      if (r.p && ((uintptr_t)r.p % (uintptr_t)r.align) != 0)
        return set_error(MUSE_ERR_INVALID_ARG, "%s is not %d-byte aligned", r.name, r.align);
  for (size_t i = 0; i < outputs.size(); ++i) {
    for (const Range &in : inputs)
      if (ranges_overlap(outputs[i], in))
        return set_error(MUSE_ERR_INVALID_ARG, "output %s overlaps input %s", outputs[i].name, in.name);
    for (size_t j = i + 1; j < outputs.size(); ++j)
      if (ranges_overlap(outputs[i], outputs[j]))
        return set_error(MUSE_ERR_INVALID_ARG, "outputs %s and %s overlap", outputs[i].name, outputs[j].name);
  }
  return MUSE_OK;
}

bool finite(float x) { return std::isfinite(x); }

muse_status check_params(const muse_attn_params *p) {
  if (!p) return set_error(MUSE_ERR_INVALID_ARG, "params is NULL");
  if (p->head_dim <= 0 || (p->head_dim & 1))
    return set_error(MUSE_ERR_INVALID_ARG, "head_dim %d must be positive and even", p->head_dim);
  if (p->num_heads <= 0 || p->num_key_value_heads <= 0)
    return set_error(MUSE_ERR_INVALID_ARG, "num_heads %d / num_key_value_heads %d must be positive",
                     p->num_heads, p->num_key_value_heads);
  if (p->num_heads % p->num_key_value_heads)
    return set_error(MUSE_ERR_INVALID_ARG, "num_heads %d is not a multiple of num_key_value_heads %d",
                     p->num_heads, p->num_key_value_heads);
  if (!finite(p->scaling) || p->scaling <= 0.0f)
    return set_error(MUSE_ERR_INVALID_ARG, "scaling must be finite and > 0");
  if (!finite(p->query_scale)) return set_error(MUSE_ERR_INVALID_ARG, "query_scale must be finite");
  if (!finite(p->qk_eps) || p->qk_eps < 0.0f || !finite(p->out_eps) || p->out_eps < 0.0f)
    return set_error(MUSE_ERR_INVALID_ARG, "qk_eps/out_eps must be finite and >= 0");
  if (!finite(p->gain_center)) return set_error(MUSE_ERR_INVALID_ARG, "gain_center must be finite");
  if (p->bidirectional && p->sliding_window > 0)
    return set_error(MUSE_ERR_INVALID_ARG, "a sliding window applies to causal attention only");
  if (p->kv_split < 0) return set_error(MUSE_ERR_INVALID_ARG, "kv_split %d must be >= 0", p->kv_split);
  if (p->head_dim != 64 && p->head_dim != 128)
    return set_error(MUSE_ERR_UNSUPPORTED, "head_dim %d: kernels exist for 64 and 128", p->head_dim);
  return MUSE_OK;
}

// Checks the layout and fills g.  With MUSE_DEBUG_VALIDATE=1 and `device_check`
// the device cu_seqlens is copied back and validated (that synchronises the
// stream).
muse_status check_layout(const muse_layout *l, const muse_attn_params *p, hipStream_t stream, Geometry *g,
                         bool device_check = true) {
  if (!l) return set_error(MUSE_ERR_INVALID_ARG, "layout is NULL");
  g->d = p->head_dim;
  g->hq = p->num_heads;
  g->hkv = p->num_key_value_heads;
  g->group = g->hq / g->hkv;
  if (l->cu_seqlens) {
    if (l->num_segments < 1) return set_error(MUSE_ERR_INVALID_ARG, "THD num_segments %d < 1", l->num_segments);
    if (l->total_tokens < 0 || l->max_seqlen < 0)
      return set_error(MUSE_ERR_INVALID_ARG, "THD total_tokens/max_seqlen must be >= 0");
    if (l->max_seqlen > l->total_tokens)
      return set_error(MUSE_ERR_INVALID_ARG, "max_seqlen %d > total_tokens %d", l->max_seqlen, l->total_tokens);
    if (l->total_tokens > 0 && l->max_seqlen < 1)
      return set_error(MUSE_ERR_INVALID_ARG, "max_seqlen must be >= 1 when total_tokens > 0");
    if (l->attention_mask)
      return set_error(MUSE_ERR_INVALID_ARG, "attention_mask is for BSHD; packed THD carries no padding");
    g->thd = true;
    g->n_tokens = l->total_tokens;
    g->nseg = l->num_segments;
    g->maxlen = l->max_seqlen;
    if (device_check && debug_validate_enabled()) {
      const muse_status s = debug_check_cu_seqlens(l, stream);
      if (s != MUSE_OK) return s;
    }
  } else {
    if (l->batch < 0 || l->seqlen < 0)
      return set_error(MUSE_ERR_INVALID_ARG, "BSHD batch %d / seqlen %d must be >= 0", l->batch, l->seqlen);
    g->thd = false;
    g->n_tokens = (int64_t)l->batch * l->seqlen;
    g->nseg = l->batch;
    g->maxlen = l->seqlen;
  }
  if (g->n_tokens * (g->hq + g->hkv) > INT32_MAX)
    return set_error(MUSE_ERR_UNSUPPORTED, "%lld tokens x %d heads exceed the 2^31 row limit",
                     (long long)g->n_tokens, g->hq + g->hkv);
  return MUSE_OK;
}

TokenLayout token_layout(const muse_layout *l, const Geometry &g) {
  TokenLayout t;
  t.n_tokens = (int32_t)g.n_tokens;
  t.seqlen = g.thd ? 0 : l->seqlen;
  t.seqlen_div = FastDiv(g.thd || l->seqlen < 1 ? 1u : (uint32_t)l->seqlen);
  t.cu_seqlens = g.thd ? l->cu_seqlens : nullptr;
  t.num_segments = g.nseg;
  t.position_ids = l->position_ids;
  return t;
}

Range layout_range(const muse_layout *l, const Geometry &g, int which) {
  if (which == 0) return Range{g.thd ? l->cu_seqlens : nullptr, ((int64_t)g.nseg + 1) * 4, "cu_seqlens", 4};
  if (which == 2) return Range{l->attention_mask, g.n_tokens, "attention_mask", 1};
  return Range{l->position_ids, g.n_tokens * 4, "position_ids", 4};
}

// The RoPE table rules; with MUSE_DEBUG_VALIDATE=1 explicit position_ids are
// copied back and checked against [0, n_pos) (that synchronises the stream).
muse_status check_rope_table(const muse_attn_params *p, const muse_layout *l, const Geometry &g,
                             const float *cos, const float *sin, int32_t n_pos, hipStream_t stream) {
  if (!p->use_rope || g.n_tokens == 0) return MUSE_OK;
  if (!cos || !sin) return set_error(MUSE_ERR_INVALID_ARG, "use_rope needs the cos and sin tables");
  if (n_pos < 1) return set_error(MUSE_ERR_INVALID_ARG, "n_pos %d < 1", n_pos);
  if (!l->position_ids && n_pos < g.maxlen)
    return set_error(MUSE_ERR_INVALID_ARG, "cos/sin table has %d positions, the layout needs %d", n_pos,
                     g.maxlen);
  if (l->position_ids && ((uintptr_t)l->position_ids % 4) == 0 && debug_validate_enabled())
    return debug_check_positions(l->position_ids, g.n_tokens, n_pos, stream);
  return MUSE_OK;
}

muse_status device_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return set_error(MUSE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  clear_error();
  return MUSE_OK;
}

// Workgroup shape: a workgroup holds a fixed number of (token, head) query
// columns; its heads are the largest divisor of the KV group size that fits,
// and as many whole tokens as the columns allow.
void attn_shape(int group, int *heads_per_wg, int *tok_per_wg, int *head_chunks) {
  const int cols = attn_columns_per_workgroup();
  int h = 1;
  for (int d = group < cols ? group : cols; d >= 1; --d)
    if (group % d == 0) { h = d; break; }
  *heads_per_wg = h;
  *tok_per_wg = cols / h;
  *head_chunks = group / h;
}

AttnArgs attn_args(const muse_attn_params *p, const muse_layout *l, const Geometry &g) {
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.eps = p->qk_eps;
  a.out_eps = p->out_eps;
  a.gain_center = p->gain_center;
  a.query_scale = p->query_scale;
  a.use_rope = p->use_rope ? 1 : 0;
  a.rope_v2 = p->upcast_rope ? 0 : 1;
  a.scaling = p->scaling;
  a.scale_log2 = p->scaling * 1.4426950408889634f;
  a.hq = g.hq;
  a.hkv = g.hkv;
  a.group = g.group;
  attn_shape(g.group, &a.heads_per_wg, &a.tok_per_wg, &a.head_chunks);
  a.window = p->sliding_window > 0 ? p->sliding_window : 0;
  a.bidirectional = p->bidirectional ? 1 : 0;
  a.key_valid = g.thd ? nullptr : l->attention_mask;
  a.q_blocks = (g.maxlen + a.tok_per_wg - 1) / a.tok_per_wg;
  a.kv_parts = 1;
  a.lay = token_layout(l, g);
  return a;
}

int64_t bf16_bytes(int64_t n, int h, int d) { return n * h * d * 2; }

// ---- KV split of the attention forward (flash-decoding style).  A grid
// with fewer than two work items per CU leaves CUs idle and lets its longest
// items (the last query blocks of a causal sequence) set the kernel's length;
// then each item's key tiles are cut into parts of kv_span tiles run by
// separate workgroups, combined per wave by the last part to finish.  The plan
// depends only on the params, the shape and the device's CU count, so the
// fused and unfused kernels take the same one (and stay bitwise equal).  Its
// partial slots and arrival counters live in the caller's workspace:
// [counters, padded to kWsAlign][slots].

constexpr size_t kWsAlign = 256;
size_t ws_round(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

int current_device_cus() {
  int dev = 0, c = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return c > 0 ? c : 0;
}

// The heaviest query block's key-tile count (the attention kernels' own tile
// range for each query block of the longest segment).
int max_item_tiles(int q_blocks, int tok_per_wg, int window, bool bidir, int maxlen) {
  const int bn = attn_keys_per_tile();
  int best = 0;
  for (int qb = 0; qb < q_blocks; ++qb) {
    const int q0 = qb * tok_per_wg;
    if (q0 >= maxlen) break;
    const int q1 = std::min(q0 + tok_per_wg, maxlen);
    const int lo = window > 0 && !bidir ? std::max(0, q0 - window + 1) : 0;
    const int hi = (bidir ? maxlen : q1) - 1;
    best = std::max(best, hi / bn - lo / bn + 1);
  }
  return best;
}

// Parts and span (steps per part) of a grid of `items` work items whose
// heaviest takes `steps` tile steps, with `per_cu` workgroups resident per CU;
// the automatic policy aims at `fill_x2` / 2 workgroups per resident slot.
void split_plan(int policy, int64_t items, int steps, int per_cu, int max_auto, int fill_x2, int *parts,
                int *span) {
  *parts = 1;
  *span = 0;
  if (policy == 1 || steps < 2) return;
  int n;
  if (policy >= 2) {
    n = std::min(std::min(policy, steps), kMaxKvParts);
  } else {
    const int cus = current_device_cus();
    const int64_t slots = (int64_t)cus * per_cu;
    if (cus <= 0 || items >= slots) return;
    // parts of at least 4 steps, so a part's prologue stays small beside its
    // tile loop
    n = (int)std::min<int64_t>(max_auto, (fill_x2 * slots + 2 * items - 1) / (2 * items));
    n = std::min(n, steps / 4);
  }
  if (n < 2) return;
  const int sp = (steps + n - 1) / n;
  n = (steps + sp - 1) / sp;
  if (n < 2) return;
  *parts = n;
  *span = sp;
}

// A split's plan and the workspace it needs: counters first, then slots.
struct SplitNeed {
  int parts = 1, span = 0;
  int64_t counters = 0;   // uint32 arrival counters (items x waves)
  size_t slot_bytes = 0;  // partial slots
  size_t bytes() const { return parts > 1 ? ws_round((size_t)counters * 4) + slot_bytes : 0; }
};

SplitNeed fwd_split_need(const AttnArgs &a, const Geometry &g, int policy) {
  SplitNeed n;
  const int64_t items = (int64_t)a.q_blocks * g.nseg * a.hkv * a.head_chunks;
  split_plan(policy, items, max_item_tiles(a.q_blocks, a.tok_per_wg, a.window, a.bidirectional != 0, g.maxlen), 2,
             4, 3, &n.parts, &n.span);
  if (n.parts < 2) return n;
  const int nw = attn_waves_per_workgroup();
  // per slot and lane: the wave's O fragment (D/32 tiles of 16) plus reference and sum
  const size_t slot = (size_t)(g.d / 32 * 16 + 2) * 64 * sizeof(float);
  n.counters = items * nw;
  n.slot_bytes = (size_t)items * n.parts * nw * slot;
  return n;
}

// The heaviest 128-key block's (query tile, head) steps in the dK/dV kernel.
int max_dkv_steps(const AttnBwdArgs &a, int maxlen) {
  const int kpw = attn_bwd_keys_per_workgroup(), bn = attn_keys_per_tile();
  int best = 0;
  for (int kb = 0; kb < a.k_blocks; ++kb) {
    const int kb0 = kb * kpw;
    if (kb0 >= maxlen) break;
    const int qlo = a.bidirectional ? 0 : kb0;
    const int qhi = a.bidirectional || a.window <= 0
                        ? maxlen - 1
                        : std::min(maxlen - 1, std::min(kb0 + kpw - 1, maxlen - 1) + a.window - 1);
    best = std::max(best, (qhi / bn - qlo / bn + 1) * a.group);
  }
  return best;
}

// Splits of the two attention-backward kernels (the dQ kernel as the forward,
// the dK/dV kernel over its query steps); they run one after the other and
// share one set of slots and counters.
struct BwdSplitNeed {
  SplitNeed q, kv;
  int64_t counters = 0;
  size_t slot_bytes = 0;
  size_t bytes() const { return (q.parts > 1 || kv.parts > 1) ? ws_round((size_t)counters * 4) + slot_bytes : 0; }
};

BwdSplitNeed bwd_split_need(const AttnBwdArgs &a, const Geometry &g, int policy) {
  BwdSplitNeed n;
  const int64_t items_q = (int64_t)a.q_blocks * g.nseg * a.hkv * a.head_chunks;
  const int64_t items_k = (int64_t)a.k_blocks * g.nseg * a.hkv;
  split_plan(policy, items_q, max_item_tiles(a.q_blocks, a.tok_per_wg, a.window, a.bidirectional != 0, g.maxlen),
             2, 4, 3, &n.q.parts, &n.q.span);
  // the D = 128 dK/dV kernel runs one workgroup per CU; one round of them
  // (a 1.5-round split of the 16k/window-4096 share was 2 % slower than none)
  split_plan(policy, items_k, max_dkv_steps(a, g.maxlen), g.d == 128 ? 1 : 2, kMaxKvParts, 2, &n.kv.parts,
             &n.kv.span);
  const int nw = attn_waves_per_workgroup();
  const size_t acc_bytes = (size_t)32 * g.d * sizeof(float);   // one D x 32 fp32 accumulator per wave
  n.slot_bytes = std::max(n.q.parts > 1 ? (size_t)items_q * n.q.parts * nw * acc_bytes : 0,
                          n.kv.parts > 1 ? (size_t)items_k * n.kv.parts * nw * 2 * acc_bytes : 0);
  // at D = 128 the two roles of a dK/dV key group arrive on counters of their own
  n.counters = std::max(n.q.parts > 1 ? items_q : 0, n.kv.parts > 1 ? items_k * (g.d == 128 ? 2 : 1) : 0) * nw;
  return n;
}

muse_status check_workspace(void *ws, size_t have, size_t need) {
  if (need == 0) return MUSE_OK;
  if (!ws) return set_error(MUSE_ERR_INVALID_ARG, "workspace is NULL (%zu bytes needed)", need);
  if ((uintptr_t)ws % 16) return set_error(MUSE_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (have < need) return set_error(MUSE_ERR_INVALID_ARG, "workspace has %zu bytes, %zu needed", have, need);
  return MUSE_OK;
}

}  // namespace
}  // namespace muse

using namespace muse;

extern "C" muse_status muse_rope_cos_sin(float theta, int32_t head_dim, int32_t n_pos, float *cos_out,
                                         float *sin_out, void *stream) {
  if (!std::isfinite(theta) || theta <= 0.0f) return set_error(MUSE_ERR_INVALID_ARG, "theta must be finite and > 0");
  if (head_dim <= 0 || (head_dim & 1)) return set_error(MUSE_ERR_INVALID_ARG, "head_dim %d must be positive and even", head_dim);
  if (n_pos < 0) return set_error(MUSE_ERR_INVALID_ARG, "n_pos %d < 0", n_pos);
  if (n_pos == 0) { clear_error(); return MUSE_OK; }
  if (!cos_out || !sin_out) return set_error(MUSE_ERR_INVALID_ARG, "cos_out/sin_out is NULL");
  const int64_t bytes = (int64_t)n_pos * (head_dim / 2) * 4;
  muse_status s = check_disjoint({}, {{cos_out, bytes, "cos_out"}, {sin_out, bytes, "sin_out"}});
  if (s != MUSE_OK) return s;
  RopeTableArgs a{theta, head_dim, n_pos, cos_out, sin_out, 0};
  return device_status(launch_rope_table(a, (hipStream_t)stream), "rope table launch");
}

extern "C" muse_status muse_rope_cos_sin_2d(float theta, int32_t head_dim, int32_t grid_h, int32_t grid_w,
                                            float *cos_out, float *sin_out, void *stream) {
  if (!std::isfinite(theta) || theta <= 0.0f) return set_error(MUSE_ERR_INVALID_ARG, "theta must be finite and > 0");
  if (head_dim <= 0 || (head_dim & 3))
    return set_error(MUSE_ERR_INVALID_ARG, "head_dim %d must be a positive multiple of 4", head_dim);
  if (grid_h < 0 || grid_w < 0) return set_error(MUSE_ERR_INVALID_ARG, "grid %d x %d is negative", grid_h, grid_w);
  const int64_t n_pos = (int64_t)grid_h * grid_w;
  if (n_pos > INT32_MAX) return set_error(MUSE_ERR_INVALID_ARG, "grid %d x %d exceeds 2^31 - 1 patches", grid_h, grid_w);
  if (n_pos == 0) { clear_error(); return MUSE_OK; }
  if (!cos_out || !sin_out) return set_error(MUSE_ERR_INVALID_ARG, "cos_out/sin_out is NULL");
  const int64_t bytes = n_pos * (head_dim / 2) * 4;
  muse_status s = check_disjoint({}, {{cos_out, bytes, "cos_out"}, {sin_out, bytes, "sin_out"}});
  if (s != MUSE_OK) return s;
  RopeTableArgs a{theta, head_dim, (int32_t)n_pos, cos_out, sin_out, grid_w};
  return device_status(launch_rope_table(a, (hipStream_t)stream), "2-D rope table launch");
}

// muse_qk_norm_rope, and with table_out muse_qk_norm_rope_table (cos/sin are
// then the tables to write, theta their base).
static muse_status qk_norm_rope_impl(const muse_attn_params *p, const muse_layout *l, const void *q,
                                     const void *k, const float *q_gain, const float *k_gain, const float *cos,
                                     const float *sin, int32_t n_pos, void *q_out, void *k_out, float *q_rstd,
                                     float *k_rstd, void *stream, bool table_out, float theta) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  Geometry g;
  s = check_layout(l, p, (hipStream_t)stream, &g);
  if (s != MUSE_OK) return s;
  if (table_out) {
    if (!p->use_rope) return set_error(MUSE_ERR_INVALID_ARG, "the table is built only for use_rope");
    if (!std::isfinite(theta) || theta <= 0.0f) return set_error(MUSE_ERR_INVALID_ARG, "theta must be finite and > 0");
  }
  if ((q == nullptr) != (q_out == nullptr)) return set_error(MUSE_ERR_INVALID_ARG, "q and q_out must be given together");
  if ((k == nullptr) != (k_out == nullptr)) return set_error(MUSE_ERR_INVALID_ARG, "k and k_out must be given together");
  if (!q && !k) return set_error(MUSE_ERR_INVALID_ARG, "neither q nor k given");
  if (!q && q_rstd) return set_error(MUSE_ERR_INVALID_ARG, "q_rstd given without q");
  if (!k && k_rstd) return set_error(MUSE_ERR_INVALID_ARG, "k_rstd given without k");
  if (p->skip_qk_norm && (q_gain || k_gain || q_rstd || k_rstd))
    return set_error(MUSE_ERR_INVALID_ARG, "skip_qk_norm takes no gains and no rstd outputs");
  s = check_rope_table(p, l, g, cos, sin, n_pos, (hipStream_t)stream);
  if (s != MUSE_OK) return s;
  const int64_t N = g.n_tokens;
  const int64_t tab = p->use_rope ? (int64_t)n_pos * (g.d / 2) * 4 : 0;
  const int64_t tab_in = table_out ? 0 : tab, tab_out = table_out ? tab : 0;
  s = check_disjoint(
      {{q, bf16_bytes(N, g.hq, g.d), "q"}, {k, bf16_bytes(N, g.hkv, g.d), "k"}, {q_gain, g.d * 4, "q_gain"},
       {k_gain, g.d * 4, "k_gain"}, {table_out ? nullptr : cos, tab_in, "cos"},
       {table_out ? nullptr : sin, tab_in, "sin"}, layout_range(l, g, 0), layout_range(l, g, 1)},
      {{q_out, bf16_bytes(N, g.hq, g.d), "q_out"}, {k_out, bf16_bytes(N, g.hkv, g.d), "k_out"},
       {q_rstd, N * g.hq * 4, "q_rstd", 4}, {k_rstd, N * g.hkv * 4, "k_rstd", 4},
       {table_out ? cos : nullptr, tab_out, "cos_out"}, {table_out ? sin : nullptr, tab_out, "sin_out"}});
  if (s != MUSE_OK) return s;
  if (N == 0) { clear_error(); return MUSE_OK; }
  QkNormArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.q_out = (uint16_t *)q_out;
  a.k_out = (uint16_t *)k_out;
  a.q_rstd = q_rstd;
  a.k_rstd = k_rstd;
  a.q_gain = q_gain;
  a.k_gain = k_gain;
  a.cos_tab = cos;
  a.sin_tab = sin;
  a.n_pos = n_pos;
  a.hq = g.hq;
  a.hkv = g.hkv;
  a.hq_div = FastDiv((uint32_t)g.hq);
  a.hkv_div = FastDiv((uint32_t)g.hkv);
  a.q_rows = q ? (int32_t)(N * g.hq) : 0;
  a.k_rows = k ? (int32_t)(N * g.hkv) : 0;
  a.eps = p->qk_eps;
  a.gain_center = p->gain_center;
  a.query_scale = p->query_scale;
  a.use_rope = p->use_rope ? 1 : 0;
  a.rope_v2 = p->upcast_rope ? 0 : 1;
  a.skip_norm = p->skip_qk_norm ? 1 : 0;
  if (table_out) {
    a.cos_tab = a.sin_tab = nullptr;
    a.theta = theta;
    a.cos_out = const_cast<float *>(cos);
    a.sin_out = const_cast<float *>(sin);
  }
  a.lay = token_layout(l, g);
  return device_status(launch_qk_norm_rope(g.d, a, (hipStream_t)stream), "qk_norm_rope launch");
}

extern "C" muse_status muse_qk_norm_rope(const muse_attn_params *p, const muse_layout *l, const void *q,
                                         const void *k, const float *q_gain, const float *k_gain,
                                         const float *cos, const float *sin, int32_t n_pos, void *q_out,
                                         void *k_out, float *q_rstd, float *k_rstd, void *stream) {
  return qk_norm_rope_impl(p, l, q, k, q_gain, k_gain, cos, sin, n_pos, q_out, k_out, q_rstd, k_rstd, stream,
                           false, 0.0f);
}

extern "C" muse_status muse_qk_norm_rope_table(const muse_attn_params *p, const muse_layout *l, const void *q,
                                               const void *k, const float *q_gain, const float *k_gain,
                                               float theta, int32_t n_pos, float *cos_out, float *sin_out,
                                               void *q_out, void *k_out, float *q_rstd, float *k_rstd,
                                               void *stream) {
  return qk_norm_rope_impl(p, l, q, k, q_gain, k_gain, cos_out, sin_out, n_pos, q_out, k_out, q_rstd, k_rstd,
                           stream, true, theta);
}

// Points a at the forward split's slots in the workspace and zeroes the
// arrival counters on the stream (a workspace reused for another shape may
// hold old slot values where this call's counters sit).
static muse_status bind_fwd_split(AttnArgs &a, const SplitNeed &n, void *ws, hipStream_t stream) {
  a.kv_parts = n.parts;
  a.kv_span = n.span;
  if (n.parts < 2) return MUSE_OK;
  a.part_cnt = (uint32_t *)ws;
  a.part_o = (float *)((char *)ws + ws_round((size_t)n.counters * 4));
  return device_status(launch_zero_u32(a.part_cnt, n.counters, stream), "KV-split counter reset");
}

extern "C" muse_status muse_attn_fwd_workspace_size(const muse_attn_params *p, const muse_layout *l,
                                                    size_t *bytes) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  Geometry g;
  s = check_layout(l, p, nullptr, &g, false);
  if (s != MUSE_OK) return s;
  if (!bytes) return set_error(MUSE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = g.n_tokens == 0 ? 0 : fwd_split_need(attn_args(p, l, g), g, p->kv_split).bytes();
  clear_error();
  return MUSE_OK;
}

extern "C" muse_status muse_gqa_attn_fwd(const muse_attn_params *p, const muse_layout *l, const void *q_hat,
                                         const void *k_hat, const void *v, void *o, float *lse, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  Geometry g;
  s = check_layout(l, p, (hipStream_t)stream, &g);
  if (s != MUSE_OK) return s;
  const int64_t N = g.n_tokens;
  if (N > 0 && (!q_hat || !k_hat || !v || !o))
    return set_error(MUSE_ERR_INVALID_ARG, "q_hat, k_hat, v and o are required");
  AttnArgs a = attn_args(p, l, g);
  const SplitNeed split = N > 0 ? fwd_split_need(a, g, p->kv_split) : SplitNeed{};
  s = check_disjoint({{q_hat, bf16_bytes(N, g.hq, g.d), "q_hat"}, {k_hat, bf16_bytes(N, g.hkv, g.d), "k_hat"},
                      {v, bf16_bytes(N, g.hkv, g.d), "v"}, layout_range(l, g, 0), layout_range(l, g, 1),
                      layout_range(l, g, 2)},
                     {{o, bf16_bytes(N, g.hq, g.d), "o"}, {lse, N * g.hq * 4, "lse", 4},
                      {split.bytes() ? workspace : nullptr, (int64_t)split.bytes(), "workspace"}});
  if (s != MUSE_OK) return s;
  if ((s = check_workspace(workspace, workspace_bytes, split.bytes())) != MUSE_OK) return s;
  if (N == 0) { clear_error(); return MUSE_OK; }
  a.q = (const uint16_t *)q_hat;
  a.k = (const uint16_t *)k_hat;
  a.v = (const uint16_t *)v;
  a.o = (uint16_t *)o;
  a.lse = lse;
  if ((s = bind_fwd_split(a, split, workspace, (hipStream_t)stream)) != MUSE_OK) return s;
  return device_status(launch_attn_fwd(g.d, false, a, (hipStream_t)stream), "attention launch");
}

extern "C" muse_status muse_out_norm_gate(const muse_attn_params *p, const muse_layout *l, const void *o,
                                          const void *gate, void *out, float *o_rstd, void *stream) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  Geometry g;
  s = check_layout(l, p, (hipStream_t)stream, &g);
  if (s != MUSE_OK) return s;
  const int64_t N = g.n_tokens;
  if (N > 0 && (!o || !gate || !out)) return set_error(MUSE_ERR_INVALID_ARG, "o, gate and out are required");
  s = check_disjoint({{o, bf16_bytes(N, g.hq, g.d), "o"}, {gate, bf16_bytes(N, g.hq, g.d), "gate"}},
                     {{out, bf16_bytes(N, g.hq, g.d), "out"}, {o_rstd, N * g.hq * 4, "o_rstd", 4}});
  if (s != MUSE_OK) return s;
  if (N == 0) { clear_error(); return MUSE_OK; }
  OutGateArgs a{(const uint16_t *)o, (const uint16_t *)gate, (uint16_t *)out, o_rstd, N * g.hq, p->out_eps};
  return device_status(launch_out_norm_gate(g.d, a, (hipStream_t)stream), "out_norm_gate launch");
}

extern "C" muse_status muse_attn_fused_fwd(const muse_attn_params *p, const muse_layout *l, const void *q,
                                           const void *k_hat, const void *v, const void *gate,
                                           const float *q_gain, const float *cos, const float *sin,
                                           int32_t n_pos, void *out, float *lse, void *workspace,
                                           size_t workspace_bytes, void *stream) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  if (p->skip_qk_norm) return set_error(MUSE_ERR_UNSUPPORTED, "the fused core normalises Q; skip_qk_norm is for muse_qk_norm_rope");
  Geometry g;
  s = check_layout(l, p, (hipStream_t)stream, &g);
  if (s != MUSE_OK) return s;
  const int64_t N = g.n_tokens;
  if (N > 0 && (!q || !k_hat || !v || !gate || !out))
    return set_error(MUSE_ERR_INVALID_ARG, "q, k_hat, v, gate and out are required");
  s = check_rope_table(p, l, g, cos, sin, n_pos, (hipStream_t)stream);
  if (s != MUSE_OK) return s;
  AttnArgs a = attn_args(p, l, g);
  const SplitNeed split = N > 0 ? fwd_split_need(a, g, p->kv_split) : SplitNeed{};
  const int64_t tab = p->use_rope ? (int64_t)n_pos * (g.d / 2) * 4 : 0;
  s = check_disjoint({{q, bf16_bytes(N, g.hq, g.d), "q"}, {k_hat, bf16_bytes(N, g.hkv, g.d), "k_hat"},
                      {v, bf16_bytes(N, g.hkv, g.d), "v"}, {gate, bf16_bytes(N, g.hq, g.d), "gate"},
                      {q_gain, g.d * 4, "q_gain"}, {cos, tab, "cos"}, {sin, tab, "sin"},
                      layout_range(l, g, 0), layout_range(l, g, 1), layout_range(l, g, 2)},
                     {{out, bf16_bytes(N, g.hq, g.d), "out"}, {lse, N * g.hq * 4, "lse", 4},
                      {split.bytes() ? workspace : nullptr, (int64_t)split.bytes(), "workspace"}});
  if (s != MUSE_OK) return s;
  if ((s = check_workspace(workspace, workspace_bytes, split.bytes())) != MUSE_OK) return s;
  if (N == 0) { clear_error(); return MUSE_OK; }
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k_hat;
  a.v = (const uint16_t *)v;
  a.gate = (const uint16_t *)gate;
  a.o = (uint16_t *)out;
  a.lse = lse;
  a.q_gain = q_gain;
  a.cos_tab = cos;
  a.sin_tab = sin;
  a.n_pos = n_pos;
  if ((s = bind_fwd_split(a, split, workspace, (hipStream_t)stream)) != MUSE_OK) return s;
  return device_status(launch_attn_fwd(g.d, true, a, (hipStream_t)stream), "fused attention launch");
}

extern "C" muse_status muse_attn_core_fwd(const muse_attn_params *p, const muse_layout *l, const void *q,
                                          const void *k, const void *v, const void *gate, const float *q_gain,
                                          const float *k_gain, const float *cos, const float *sin, int32_t n_pos,
                                          void *k_hat_out, void *out, float *lse, void *workspace,
                                          size_t workspace_bytes, void *stream) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  if (p->skip_qk_norm) return set_error(MUSE_ERR_UNSUPPORTED, "the fused core normalises Q/K; skip_qk_norm is for muse_qk_norm_rope");
  Geometry g;
  s = check_layout(l, p, (hipStream_t)stream, &g);
  if (s != MUSE_OK) return s;
  const int64_t N = g.n_tokens;
  if (N > 0 && (!q || !k || !v || !gate || !k_hat_out || !out))
    return set_error(MUSE_ERR_INVALID_ARG, "q, k, v, gate, k_hat_out and out are required");
  s = check_rope_table(p, l, g, cos, sin, n_pos, (hipStream_t)stream);
  if (s != MUSE_OK) return s;
  const int64_t tab = p->use_rope ? (int64_t)n_pos * (g.d / 2) * 4 : 0;
  const size_t split_bytes = N > 0 ? fwd_split_need(attn_args(p, l, g), g, p->kv_split).bytes() : 0;
  s = check_disjoint(
      {{q, bf16_bytes(N, g.hq, g.d), "q"}, {k, bf16_bytes(N, g.hkv, g.d), "k"}, {v, bf16_bytes(N, g.hkv, g.d), "v"},
       {gate, bf16_bytes(N, g.hq, g.d), "gate"}, {q_gain, g.d * 4, "q_gain"}, {k_gain, g.d * 4, "k_gain"},
       {cos, tab, "cos"}, {sin, tab, "sin"}, layout_range(l, g, 0), layout_range(l, g, 1),
       layout_range(l, g, 2)},
      {{k_hat_out, bf16_bytes(N, g.hkv, g.d), "k_hat_out"}, {out, bf16_bytes(N, g.hq, g.d), "out"},
       {lse, N * g.hq * 4, "lse", 4}, {split_bytes ? workspace : nullptr, (int64_t)split_bytes, "workspace"}});
  if (s != MUSE_OK) return s;
  if ((s = check_workspace(workspace, workspace_bytes, split_bytes)) != MUSE_OK) return s;
  if (N == 0) { clear_error(); return MUSE_OK; }
  // keys: norm + gain + RoPE once per key (the K-only pass of the Q/K kernel),
  // then attention with the query prologue and the norm/gate epilogue fused.
  s = muse_qk_norm_rope(p, l, nullptr, k, nullptr, k_gain, cos, sin, n_pos, nullptr, k_hat_out, nullptr,
                        nullptr, stream);
  if (s != MUSE_OK) return s;
  return muse_attn_fused_fwd(p, l, q, k_hat_out, v, gate, q_gain, cos, sin, n_pos, out, lse, workspace,
                             workspace_bytes, stream);
}

// ---------------------------------------------------------------- backward

namespace muse {
namespace {

size_t qk_bwd_partial_bytes(const Geometry &g, bool q_gain, bool k_gain) {
  int32_t qb = 0, kb = 0;
  qk_norm_bwd_blocks(g.d, g.n_tokens * g.hq, g.n_tokens * g.hkv, &qb, &kb);
  return ws_round((size_t)(q_gain ? qb : 0) * g.d * 4) + ws_round((size_t)(k_gain ? kb : 0) * g.d * 4);
}

// Core workspace: the attention splits' region (the recomputed forward's
// and the attention backward's, used one after the other), then q_hat, k_hat,
// o, lse, d_o, delta, dq_hat, dk_hat and the gain partials.
struct CoreWs {
  size_t split, q_hat, k_hat, o, lse, d_o, delta, dq_hat, dk_hat, part, total;
};
CoreWs core_ws(const Geometry &g, size_t split_bytes) {
  CoreWs w;
  const size_t nq = (size_t)g.n_tokens * g.hq, nk = (size_t)g.n_tokens * g.hkv;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += ws_round(bytes); return at; };
  w.split = take(split_bytes);
  w.q_hat = take(nq * g.d * 2);
  w.k_hat = take(nk * g.d * 2);
  w.o = take(nq * g.d * 2);
  w.lse = take(nq * 4);
  w.d_o = take(nq * g.d * 2);
  w.delta = take(nq * 4);
  w.dq_hat = take(nq * g.d * 2);
  w.dk_hat = take(nk * g.d * 2);
  w.part = take(qk_bwd_partial_bytes(g, true, true));
  w.total = off;
  return w;
}

AttnBwdArgs attn_bwd_args(const muse_attn_params *p, const muse_layout *l, const Geometry &g) {
  AttnBwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.scaling = p->scaling;
  a.scale_log2 = p->scaling * 1.4426950408889634f;
  a.hq = g.hq;
  a.hkv = g.hkv;
  a.group = g.group;
  attn_shape(g.group, &a.heads_per_wg, &a.tok_per_wg, &a.head_chunks);
  a.window = p->sliding_window > 0 ? p->sliding_window : 0;
  a.bidirectional = p->bidirectional ? 1 : 0;
  a.key_valid = g.thd ? nullptr : l->attention_mask;
  a.q_blocks = (g.maxlen + a.tok_per_wg - 1) / a.tok_per_wg;
  const int kpw = attn_bwd_keys_per_workgroup();
  a.k_blocks = (g.maxlen + kpw - 1) / kpw;
  a.dq_parts = a.dkv_parts = 1;
  a.lay = token_layout(l, g);
  return a;
}

// Split region of muse_attn_core_bwd: its forward recompute (when O and LSE
// are not given) and its attention backward take turns in it.
size_t core_split_bytes(const muse_attn_params *p, const muse_layout *l, const Geometry &g) {
  if (g.n_tokens == 0) return 0;
  return std::max(fwd_split_need(attn_args(p, l, g), g, p->kv_split).bytes(),
                  bwd_split_need(attn_bwd_args(p, l, g), g, p->kv_split).bytes());
}

// Points a at the backward split's slots and zeroes its arrival counters on
// the stream.
muse_status bind_bwd_split(AttnBwdArgs &a, const BwdSplitNeed &n, void *ws, hipStream_t stream) {
  a.dq_parts = n.q.parts;
  a.dq_span = n.q.span;
  a.dkv_parts = n.kv.parts;
  a.dkv_span = n.kv.span;
  if (n.bytes() == 0) return MUSE_OK;
  a.part_cnt = (uint32_t *)ws;
  a.part_acc = (float *)((char *)ws + ws_round((size_t)n.counters * 4));
  return device_status(launch_zero_u32(a.part_cnt, n.counters, stream), "attention-backward split counter reset");
}

}  // namespace
}  // namespace muse

extern "C" muse_status muse_out_norm_gate_bwd(const muse_attn_params *p, const muse_layout *l, const void *o,
                                              const void *gate, const void *dout, void *d_o, void *dgate,
                                              float *delta, void *stream) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  Geometry g;
  s = check_layout(l, p, (hipStream_t)stream, &g);
  if (s != MUSE_OK) return s;
  const int64_t N = g.n_tokens;
  if (N > 0 && (!o || !gate || !dout || !d_o || !dgate || !delta))
    return set_error(MUSE_ERR_INVALID_ARG, "o, gate, dout, d_o, dgate and delta are required");
  const int64_t tb = bf16_bytes(N, g.hq, g.d);
  s = check_disjoint({{o, tb, "o"}, {gate, tb, "gate"}, {dout, tb, "dout"}},
                     {{d_o, tb, "d_o"}, {dgate, tb, "dgate"}, {delta, N * g.hq * 4, "delta", 4}});
  if (s != MUSE_OK) return s;
  if (N == 0) { clear_error(); return MUSE_OK; }
  OutGateBwdArgs a{(const uint16_t *)o, (const uint16_t *)gate, (const uint16_t *)dout, (uint16_t *)d_o,
                   (uint16_t *)dgate, delta, N * g.hq, p->out_eps};
  return device_status(launch_out_norm_gate_bwd(g.d, a, (hipStream_t)stream), "out_norm_gate_bwd launch");
}

extern "C" muse_status muse_attn_bwd_delta(const muse_attn_params *p, const muse_layout *l, const void *o,
                                           const void *d_o, float *delta, void *stream) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  Geometry g;
  s = check_layout(l, p, (hipStream_t)stream, &g);
  if (s != MUSE_OK) return s;
  const int64_t N = g.n_tokens;
  if (N > 0 && (!o || !d_o || !delta)) return set_error(MUSE_ERR_INVALID_ARG, "o, d_o and delta are required");
  const int64_t tb = bf16_bytes(N, g.hq, g.d);
  s = check_disjoint({{o, tb, "o"}, {d_o, tb, "d_o"}}, {{delta, N * g.hq * 4, "delta", 4}});
  if (s != MUSE_OK) return s;
  if (N == 0) { clear_error(); return MUSE_OK; }
  OutGateBwdArgs a{(const uint16_t *)o, nullptr, (const uint16_t *)d_o, nullptr, nullptr, delta, N * g.hq, 0.0f};
  return device_status(launch_out_norm_gate_bwd(g.d, a, (hipStream_t)stream), "attention delta launch");
}

extern "C" muse_status muse_gqa_attn_bwd_workspace_size(const muse_attn_params *p, const muse_layout *l,
                                                        size_t *bytes) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  Geometry g;
  s = check_layout(l, p, nullptr, &g, false);
  if (s != MUSE_OK) return s;
  if (!bytes) return set_error(MUSE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = g.n_tokens == 0 ? 0 : bwd_split_need(attn_bwd_args(p, l, g), g, p->kv_split).bytes();
  clear_error();
  return MUSE_OK;
}

extern "C" muse_status muse_gqa_attn_bwd(const muse_attn_params *p, const muse_layout *l, const void *q_hat,
                                         const void *k_hat, const void *v, const void *d_o, const float *lse,
                                         const float *delta, void *dq_hat, void *dk_hat, void *dv, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  Geometry g;
  s = check_layout(l, p, (hipStream_t)stream, &g);
  if (s != MUSE_OK) return s;
  const int64_t N = g.n_tokens;
  if (N > 0 && (!q_hat || !k_hat || !v || !d_o || !lse || !delta || !dq_hat || !dk_hat || !dv))
    return set_error(MUSE_ERR_INVALID_ARG, "every tensor of the attention backward is required");
  AttnBwdArgs a = attn_bwd_args(p, l, g);
  const BwdSplitNeed split = N > 0 ? bwd_split_need(a, g, p->kv_split) : BwdSplitNeed{};
  const int64_t qb = bf16_bytes(N, g.hq, g.d), kb = bf16_bytes(N, g.hkv, g.d);
  s = check_disjoint({{q_hat, qb, "q_hat"}, {k_hat, kb, "k_hat"}, {v, kb, "v"}, {d_o, qb, "d_o"},
                      {lse, N * g.hq * 4, "lse", 4}, {delta, N * g.hq * 4, "delta", 4}, layout_range(l, g, 0),
                      layout_range(l, g, 1), layout_range(l, g, 2)},
                     {{dq_hat, qb, "dq_hat"}, {dk_hat, kb, "dk_hat"}, {dv, kb, "dv"},
                      {split.bytes() ? workspace : nullptr, (int64_t)split.bytes(), "workspace"}});
  if (s != MUSE_OK) return s;
  if ((s = check_workspace(workspace, workspace_bytes, split.bytes())) != MUSE_OK) return s;
  if (N == 0) { clear_error(); return MUSE_OK; }
  a.q = (const uint16_t *)q_hat;
  a.k = (const uint16_t *)k_hat;
  a.v = (const uint16_t *)v;
  a.d_o = (const uint16_t *)d_o;
  a.lse = lse;
  a.delta = delta;
  a.dq = (uint16_t *)dq_hat;
  a.dk = (uint16_t *)dk_hat;
  a.dv = (uint16_t *)dv;
  if ((s = bind_bwd_split(a, split, workspace, (hipStream_t)stream)) != MUSE_OK) return s;
  return device_status(launch_attn_bwd(g.d, a, (hipStream_t)stream), "attention backward launch");
}

extern "C" muse_status muse_qk_norm_rope_bwd_workspace_size(const muse_attn_params *p, const muse_layout *l,
                                                            size_t *bytes) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  Geometry g;
  s = check_layout(l, p, nullptr, &g, false);
  if (s != MUSE_OK) return s;
  if (!bytes) return set_error(MUSE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = p->skip_qk_norm ? 0 : qk_bwd_partial_bytes(g, true, true);
  clear_error();
  return MUSE_OK;
}

static muse_status qk_norm_rope_bwd_impl(const muse_attn_params *p, const muse_layout *l, const void *q,
                                             const void *k, const float *q_gain, const float *k_gain,
                                             const float *cos, const float *sin, int32_t n_pos, const void *dq_hat,
                                             const void *dk_hat, void *dq, void *dk, float *dq_gain, float *dk_gain,
                                             void *workspace, size_t workspace_bytes, void *stream,
                                             bool static_scratch) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  Geometry g;
  s = check_layout(l, p, (hipStream_t)stream, &g);
  if (s != MUSE_OK) return s;
  const bool has_q = q || dq_hat || dq, has_k = k || dk_hat || dk;
  if (has_q && !(q && dq_hat && dq)) return set_error(MUSE_ERR_INVALID_ARG, "q, dq_hat and dq must be given together");
  if (has_k && !(k && dk_hat && dk)) return set_error(MUSE_ERR_INVALID_ARG, "k, dk_hat and dk must be given together");
  if (!has_q && !has_k) return set_error(MUSE_ERR_INVALID_ARG, "neither q nor k given");
  if ((q_gain != nullptr) != (dq_gain != nullptr) || (k_gain != nullptr) != (dk_gain != nullptr))
    return set_error(MUSE_ERR_INVALID_ARG, "a gain gradient is given exactly when its gain is");
  if ((q_gain && !has_q) || (k_gain && !has_k))
    return set_error(MUSE_ERR_INVALID_ARG, "a gain is given without its tensor");
  if (p->skip_qk_norm && (q_gain || k_gain))
    return set_error(MUSE_ERR_INVALID_ARG, "skip_qk_norm takes no gains");
  s = check_rope_table(p, l, g, cos, sin, n_pos, (hipStream_t)stream);
  if (s != MUSE_OK) return s;
  const int64_t N = g.n_tokens;
  const int64_t qb = bf16_bytes(N, g.hq, g.d), kb = bf16_bytes(N, g.hkv, g.d);
  const int64_t tab = p->use_rope ? (int64_t)n_pos * (g.d / 2) * 4 : 0;
  const size_t need = (q_gain || k_gain) ? qk_bwd_partial_bytes(g, q_gain != nullptr, k_gain != nullptr) : 0;
  if (static_scratch && need > 0) {
    // the library-held scratch of this GPU (no allocation: a static device array)
    float *ptr = nullptr;
    size_t have = 0;
    const hipError_t e = qk_norm_bwd_static_scratch(&ptr, &have);
    if (e != hipSuccess) return device_status(e, "static scratch lookup");
    if (need > have)
      return set_error(MUSE_ERR_INVALID_ARG, "the gain partial sums need %zu bytes, more than the %zu bytes "
                       "of static scratch; use muse_qk_norm_rope_bwd with a workspace", need, have);
    workspace = ptr;
    workspace_bytes = have;
  }
  s = check_disjoint({{q, qb, "q"}, {k, kb, "k"}, {q_gain, g.d * 4, "q_gain"}, {k_gain, g.d * 4, "k_gain"},
                      {cos, tab, "cos"}, {sin, tab, "sin"}, {dq_hat, qb, "dq_hat"}, {dk_hat, kb, "dk_hat"},
                      layout_range(l, g, 0), layout_range(l, g, 1)},
                     {{dq, qb, "dq"}, {dk, kb, "dk"}, {dq_gain, g.d * 4, "dq_gain"}, {dk_gain, g.d * 4, "dk_gain"},
                      {workspace, (int64_t)need, "workspace"}});
  if (s != MUSE_OK) return s;
  if ((s = check_workspace(workspace, workspace_bytes, need)) != MUSE_OK) return s;
  if (N == 0) { clear_error(); return MUSE_OK; }
  QkNormBwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.dq_hat = (const uint16_t *)dq_hat;
  a.dk_hat = (const uint16_t *)dk_hat;
  a.dq = (uint16_t *)dq;
  a.dk = (uint16_t *)dk;
  a.q_gain = q_gain;
  a.k_gain = k_gain;
  a.cos_tab = cos;
  a.sin_tab = sin;
  a.n_pos = n_pos;
  a.hq_div = FastDiv((uint32_t)g.hq);
  a.hkv_div = FastDiv((uint32_t)g.hkv);
  a.q_rows = has_q ? (int32_t)(N * g.hq) : 0;
  a.k_rows = has_k ? (int32_t)(N * g.hkv) : 0;
  int32_t nqb = 0, nkb = 0;
  qk_norm_bwd_blocks(g.d, a.q_rows, a.k_rows, &nqb, &nkb);
  a.q_part = q_gain ? (float *)workspace : nullptr;
  a.k_part = k_gain ? (float *)((char *)workspace + (q_gain ? ws_round((size_t)nqb * g.d * 4) : 0)) : nullptr;
  a.dq_gain = dq_gain;
  a.dk_gain = dk_gain;
  a.eps = p->qk_eps;
  a.gain_center = p->gain_center;
  a.query_scale = p->query_scale;
  a.use_rope = p->use_rope ? 1 : 0;
  a.rope_v2 = p->upcast_rope ? 0 : 1;
  a.skip_norm = p->skip_qk_norm ? 1 : 0;
  a.lay = token_layout(l, g);
  return device_status(launch_qk_norm_rope_bwd(g.d, a, (hipStream_t)stream), "qk_norm_rope_bwd launch");
}


extern "C" muse_status muse_qk_norm_rope_bwd(const muse_attn_params *p, const muse_layout *l, const void *q,
                                             const void *k, const float *q_gain, const float *k_gain,
                                             const float *cos, const float *sin, int32_t n_pos, const void *dq_hat,
                                             const void *dk_hat, void *dq, void *dk, float *dq_gain, float *dk_gain,
                                             void *workspace, size_t workspace_bytes, void *stream) {
  return qk_norm_rope_bwd_impl(p, l, q, k, q_gain, k_gain, cos, sin, n_pos, dq_hat, dk_hat, dq, dk, dq_gain,
                               dk_gain, workspace, workspace_bytes, stream, false);
}

extern "C" muse_status muse_qk_norm_rope_bwd_static(const muse_attn_params *p, const muse_layout *l,
                                                    const void *q, const void *k, const float *q_gain,
                                                    const float *k_gain, const float *cos, const float *sin,
                                                    int32_t n_pos, const void *dq_hat, const void *dk_hat, void *dq,
                                                    void *dk, float *dq_gain, float *dk_gain, void *stream) {
  return qk_norm_rope_bwd_impl(p, l, q, k, q_gain, k_gain, cos, sin, n_pos, dq_hat, dk_hat, dq, dk, dq_gain,
                               dk_gain, nullptr, 0, stream, true);
}

extern "C" muse_status muse_attn_core_bwd_workspace_size(const muse_attn_params *p, const muse_layout *l,
                                                         size_t *bytes) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  Geometry g;
  s = check_layout(l, p, nullptr, &g, false);
  if (s != MUSE_OK) return s;
  if (!bytes) return set_error(MUSE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = core_ws(g, core_split_bytes(p, l, g)).total;
  clear_error();
  return MUSE_OK;
}

extern "C" muse_status muse_attn_core_bwd(const muse_attn_params *p, const muse_layout *l, const void *q,
                                          const void *k, const void *v, const void *gate, const float *q_gain,
                                          const float *k_gain, const float *cos, const float *sin, int32_t n_pos,
                                          const void *o, const float *lse, const void *dout, void *dq, void *dk,
                                          void *dv, void *dgate, float *dq_gain, float *dk_gain, void *workspace,
                                          size_t workspace_bytes, void *stream) {
  muse_status s = check_params(p);
  if (s != MUSE_OK) return s;
  if (p->skip_qk_norm) return set_error(MUSE_ERR_UNSUPPORTED, "the core normalises Q/K; skip_qk_norm is for muse_qk_norm_rope_bwd");
  Geometry g;
  s = check_layout(l, p, (hipStream_t)stream, &g);
  if (s != MUSE_OK) return s;
  const int64_t N = g.n_tokens;
  if (N > 0 && (!q || !k || !v || !gate || !dout || !dq || !dk || !dv || !dgate))
    return set_error(MUSE_ERR_INVALID_ARG, "q, k, v, gate, dout, dq, dk, dv and dgate are required");
  if ((o == nullptr) != (lse == nullptr))
    return set_error(MUSE_ERR_INVALID_ARG, "o and lse are given together (or both recomputed)");
  if ((q_gain != nullptr) != (dq_gain != nullptr) || (k_gain != nullptr) != (dk_gain != nullptr))
    return set_error(MUSE_ERR_INVALID_ARG, "a gain gradient is given exactly when its gain is");
  s = check_rope_table(p, l, g, cos, sin, n_pos, (hipStream_t)stream);
  if (s != MUSE_OK) return s;
  const CoreWs w = core_ws(g, core_split_bytes(p, l, g));
  const int64_t qb = bf16_bytes(N, g.hq, g.d), kb = bf16_bytes(N, g.hkv, g.d);
  const int64_t tab = p->use_rope ? (int64_t)n_pos * (g.d / 2) * 4 : 0;
  s = check_disjoint({{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {gate, qb, "gate"}, {q_gain, g.d * 4, "q_gain"},
                      {k_gain, g.d * 4, "k_gain"}, {cos, tab, "cos"}, {sin, tab, "sin"}, {o, qb, "o"},
                      {lse, N * g.hq * 4, "lse", 4}, {dout, qb, "dout"}, layout_range(l, g, 0),
                      layout_range(l, g, 1), layout_range(l, g, 2)},
                     {{dq, qb, "dq"}, {dk, kb, "dk"}, {dv, kb, "dv"}, {dgate, qb, "dgate"},
                      {dq_gain, g.d * 4, "dq_gain"}, {dk_gain, g.d * 4, "dk_gain"},
                      {workspace, (int64_t)w.total, "workspace"}});
  if (s != MUSE_OK) return s;
  if ((s = check_workspace(workspace, workspace_bytes, w.total)) != MUSE_OK) return s;
  if (N == 0) { clear_error(); return MUSE_OK; }
  char *ws = (char *)workspace;
  void *q_hat = ws + w.q_hat, *k_hat = ws + w.k_hat;
  // forward recompute: Q/K norm + RoPE (and the attention output when not kept)
  s = muse_qk_norm_rope(p, l, q, k, q_gain, k_gain, cos, sin, n_pos, q_hat, k_hat, nullptr, nullptr, stream);
  if (s != MUSE_OK) return s;
  if (!o) {
    o = ws + w.o;
    lse = (const float *)(ws + w.lse);
    s = muse_gqa_attn_fwd(p, l, q_hat, k_hat, v, (void *)o, (float *)lse, ws + w.split, w.q_hat - w.split,
                          stream);
    if (s != MUSE_OK) return s;
  }
  void *d_o = ws + w.d_o, *dq_hat = ws + w.dq_hat, *dk_hat = ws + w.dk_hat;
  float *delta = (float *)(ws + w.delta);
  s = muse_out_norm_gate_bwd(p, l, o, gate, dout, d_o, dgate, delta, stream);
  if (s != MUSE_OK) return s;
  s = muse_gqa_attn_bwd(p, l, q_hat, k_hat, v, d_o, lse, delta, dq_hat, dk_hat, dv, ws + w.split,
                        w.q_hat - w.split, stream);
  if (s != MUSE_OK) return s;
  return muse_qk_norm_rope_bwd(p, l, q, k, q_gain, k_gain, cos, sin, n_pos, dq_hat, dk_hat, dq, dk, dq_gain,
                               dk_gain, ws + w.part, w.total - w.part, stream);
}
