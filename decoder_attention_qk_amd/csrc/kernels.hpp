// Kernel argument blocks and launchers (internal to libmuseattn).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"

namespace muse {

// Where each token sits: its row/segment and its RoPE position.
struct TokenLayout {
  int32_t n_tokens;              // N
  int32_t seqlen;                // BSHD row length (cu_seqlens == nullptr)
  FastDiv seqlen_div;            // division by seqlen (BSHD)
  const int32_t *cu_seqlens;     // THD boundaries [num_segments + 1], or nullptr
  int32_t num_segments;          // THD segments, or BSHD batch
  const int32_t *position_ids;   // explicit RoPE positions [N], or nullptr
};

struct RopeTableArgs {
  float theta;
  int32_t head_dim;
  int32_t n_pos;
  float *cos_out;
  float *sin_out;
  int32_t grid_w;          // > 0: 2-D table of a row-major grid of n_pos / grid_w rows
};

struct QkNormArgs {
  const uint16_t *q;       // [N, Hq, D] or nullptr
  const uint16_t *k;       // [N, Hkv, D] or nullptr
  uint16_t *q_out;
  uint16_t *k_out;
  float *q_rstd;           // [N, Hq] or nullptr
  float *k_rstd;           // [N, Hkv] or nullptr
  const float *q_gain;     // [D] or nullptr
  const float *k_gain;     // [D] or nullptr
  const float *cos_tab;    // [n_pos, D/2]
  const float *sin_tab;
  int32_t n_pos;
  int32_t hq, hkv;
  FastDiv hq_div, hkv_div;
  int32_t q_rows;          // N * Hq when q is processed, else 0 (< 2^31)
  int32_t k_rows;          // N * Hkv when k is processed, else 0 (< 2^31)
  int32_t q_blocks;        // set by the launcher: blocks given to Q rows (the rest take K rows)
  float eps, gain_center, query_scale;
  int32_t use_rope;
  int32_t rope_v2;         // rotation in the Q/K dtype (upcast_rope == 0)
  int32_t skip_norm;       // scale/rotate only: no RMSNorm, no gain
  // table mode (cos_out != nullptr): each block evaluates the cos/sin rows of
  // its rows' token positions (rope_entry, as the table kernel) instead of
  // reading cos_tab/sin_tab, uses them, and writes them to cos_out/sin_out
  float theta;
  float *cos_out;
  float *sin_out;
  TokenLayout lay;
};

struct OutGateArgs {
  const uint16_t *o;       // [N, Hq, D]
  const uint16_t *gate;    // [N, Hq, D]
  uint16_t *out;           // [N, Hq, D]
  float *o_rstd;           // [N, Hq] or nullptr
  int64_t rows;            // N * Hq
  float eps;
};

// Backward of the output norm + gate: d_o, dgate and delta = rowsum(d_o * o);
// with gate == nullptr only delta = rowsum(dout * o) is formed (dout is d_o).
struct OutGateBwdArgs {
  const uint16_t *o;       // [N, Hq, D]
  const uint16_t *gate;    // [N, Hq, D] or nullptr (delta only)
  const uint16_t *dout;    // [N, Hq, D]
  uint16_t *d_o;           // [N, Hq, D] (unused in delta-only mode)
  uint16_t *dgate;         // [N, Hq, D] (unused in delta-only mode)
  float *delta;            // [N, Hq]
  int64_t rows;            // N * Hq
  float eps;
};

// Backward of the Q/K norm + query scale + RoPE.  Blocks [0, q_blocks) take
// Q rows, the rest K rows; each block walks its rows with a fixed stride and
// writes one partial gain gradient per column (part[block][D]), summed in a
// fixed order by the reduce kernel.
struct QkNormBwdArgs {
  const uint16_t *q, *k;            // raw inputs (re-normalised here)
  const uint16_t *dq_hat, *dk_hat;  // gradients of the rotated outputs
  uint16_t *dq, *dk;
  const float *q_gain, *k_gain;     // nullptr: no gain
  float *q_part, *k_part;           // [blocks, D] partial gain gradients (nullptr: no gain)
  float *dq_gain, *dk_gain;         // [D] gain gradients (with their partial buffers)
  const float *cos_tab, *sin_tab;
  int32_t n_pos;
  FastDiv hq_div, hkv_div;
  int32_t q_rows, k_rows;
  int32_t q_blocks, k_blocks;       // set by the launcher
  float eps, gain_center, query_scale;
  int32_t use_rope, skip_norm;
  int32_t rope_v2;                  // the forward rotated with bf16 cos/sin (upcast_rope == 0)
  TokenLayout lay;
};

struct AttnArgs {
  const uint16_t *q;       // fused: raw Q; otherwise normalised, rotated Q
  const uint16_t *k;       // normalised, rotated K [N, Hkv, D]
  const uint16_t *v;       // [N, Hkv, D]
  const uint16_t *gate;    // fused only: [N, Hq, D]
  uint16_t *o;             // fused: gated output; otherwise attention output
  float *lse;              // [N, Hq] or nullptr
  // fused Q prologue
  const float *q_gain;
  const float *cos_tab;
  const float *sin_tab;
  int32_t n_pos;
  int32_t use_rope;
  int32_t rope_v2;         // rotation in the Q/K dtype (upcast_rope == 0)
  float eps, out_eps, gain_center, query_scale;
  // attention
  float scaling;           // softmax scale
  float scale_log2;        // scaling * log2(e)
  int32_t hq, hkv, group;  // group = hq / hkv
  int32_t heads_per_wg;    // query heads of one kv group handled by one workgroup
  int32_t head_chunks;     // group / heads_per_wg
  int32_t tok_per_wg;      // query tokens per workgroup (tok_per_wg * heads_per_wg <= columns)
  int32_t window;          // <= 0: none
  int32_t bidirectional;   // every key of the segment is visible (no causal order, no window)
  const uint8_t *key_valid;  // BSHD [batch, seqlen] token validity (0 = padded key) or nullptr
  int32_t q_blocks;        // ceil(max segment length / tok_per_wg)
  // KV split: a work item's key tiles are cut into parts of kv_span tiles,
  // each run by its own workgroup; per wave, the last part to arrive combines
  // them (kv_parts == 1: no split, the pointers below are unused).
  int32_t kv_parts;        // 1 .. kMaxKvParts
  int32_t kv_span;
  float *part_o;           // [items][kv_parts][waves] slots: O fragment, reference, sum (per lane)
  uint32_t *part_cnt;      // [items][waves] arrivals; zeroed before the launch, zero after it
  TokenLayout lay;
};

constexpr int kMaxKvParts = 8;

// Attention backward (dQ kernel and dK/dV kernel).
struct AttnBwdArgs {
  const uint16_t *q, *k, *v;   // q_hat [N, Hq, D]; k_hat, v [N, Hkv, D]
  const uint16_t *d_o;         // [N, Hq, D]
  const float *lse;            // [N, Hq] natural-log LSE of the forward
  const float *delta;          // [N, Hq] rowsum(d_o * o)
  uint16_t *dq;                // [N, Hq, D] gradient of q_hat
  uint16_t *dk, *dv;           // [N, Hkv, D]
  float scaling, scale_log2;
  int32_t hq, hkv, group;
  int32_t heads_per_wg, head_chunks, tok_per_wg;   // dQ kernel work shape (as the forward)
  int32_t window, bidirectional;
  const uint8_t *key_valid;    // BSHD token validity or nullptr
  int32_t q_blocks;            // dQ kernel: query blocks per segment
  int32_t k_blocks;            // dK/dV kernel: 128-key blocks per segment
  // Splits of small grids (1: none): the dQ kernel's key tiles and the dK/dV
  // kernel's (query tile, head) steps are cut into parts whose fp32 sums the
  // last part of each wave adds up in part order.  The kernels run one after
  // the other, so they share the slots and counters.
  int32_t dq_parts, dq_span;
  int32_t dkv_parts, dkv_span;
  float *part_acc;             // [items][parts][waves] slots of R x C x 16 x 64 floats
  uint32_t *part_cnt;          // [items][waves] arrivals; zeroed before the launch, zero after it
  TokenLayout lay;
};

hipError_t launch_rope_table(const RopeTableArgs &a, hipStream_t stream);
hipError_t launch_qk_norm_rope(int head_dim, const QkNormArgs &a, hipStream_t stream);
hipError_t launch_out_norm_gate(int head_dim, const OutGateArgs &a, hipStream_t stream);
hipError_t launch_attn_fwd(int head_dim, bool fused, const AttnArgs &a, hipStream_t stream);
// zeroes n 32-bit words (the splits' arrival counters) in stream order
hipError_t launch_zero_u32(uint32_t *p, int64_t n, hipStream_t stream);
hipError_t launch_out_norm_gate_bwd(int head_dim, const OutGateBwdArgs &a, hipStream_t stream);
// blocks the Q/K backward uses for q_rows / k_rows rows (the partial buffers' first dimension)
void qk_norm_bwd_blocks(int head_dim, int64_t q_rows, int64_t k_rows, int32_t *q_blocks, int32_t *k_blocks);
hipError_t launch_qk_norm_rope_bwd(int head_dim, const QkNormBwdArgs &a, hipStream_t stream);
// The current device's copy of the library-held scratch of the Q/K backward's
// allocation-free entry point: its address (from hipGetSymbolAddress, looked
// up once per device) and size.
hipError_t qk_norm_bwd_static_scratch(float **ptr, size_t *bytes);
hipError_t launch_attn_bwd(int head_dim, const AttnBwdArgs &a, hipStream_t stream);
int attn_bwd_keys_per_workgroup();
int attn_columns_per_workgroup();  // (token, head) query columns one attention workgroup holds
int attn_waves_per_workgroup();
int attn_keys_per_tile();

// One RoPE table entry: pair i of a head `width` wide at coordinate coord.
// The inverse frequency theta^(-2i/width) and the cosine/sine are evaluated
// in double and rounded once to binary32; the angle is the binary32 product
// of the coordinate and that frequency.  Every kernel that forms table
// entries calls this, so they agree bit for bit.
__device__ __forceinline__ float rope_inv_freq(float theta, int i, int width) {
  return (float)pow((double)theta, -2.0 * (double)i / (double)width);
}
__device__ __forceinline__ void rope_cos_sin(int coord, float inv, float &c, float &s) {
  const float ang = (float)coord * inv;
  // one shared argument reduction; the same bits as separate cos() and sin()
  // after the binary32 rounding (checked on every entry of 131072-position
  // tables at D = 64 and 128)
  double sd, cd;
  sincos((double)ang, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}
__device__ __forceinline__ void rope_entry(float theta, int i, int width, int coord, float &c, float &s) {
  rope_cos_sin(coord, rope_inv_freq(theta, i, width), c, s);
}

// Position of token t for RoPE (clamped into the table), and its segment.
__device__ __forceinline__ int find_segment(const TokenLayout &l, int t) {
  int lo = 0, hi = l.num_segments;  // invariant: cu[lo] <= t < cu[hi] for a valid layout
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (l.cu_seqlens[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Positions of a run of consecutive tokens starting at t0 (wave-uniform, so
// the segment search runs on scalar loads once per run): a token inside the
// run's first segment needs no load at all; a later one walks forward from it
// (a run crosses few boundaries).
struct PosCursor {
  int seg, start, next;   // packed layouts: t0's segment, its first token, the next segment's
};

__device__ __forceinline__ PosCursor pos_cursor(const TokenLayout &l, int t0) {
  PosCursor c{0, 0, 0};
  if (l.cu_seqlens && !l.position_ids) {
    c.seg = find_segment(l, t0);
    c.start = l.cu_seqlens[c.seg];
    c.next = l.cu_seqlens[c.seg + 1];
  }
  return c;
}

// rope_position(l, t, n_pos) for a token t >= the cursor's t0.
__device__ __forceinline__ int rope_position(const TokenLayout &l, const PosCursor &c, int t, int n_pos) {
  int p;
  if (l.position_ids) {
    p = l.position_ids[t];
  } else if (l.cu_seqlens) {
    if (t < c.next) {
      p = t - c.start;
    } else {
      int seg = c.seg + 1;
      while (seg + 1 < l.num_segments && l.cu_seqlens[seg + 1] <= t) ++seg;
      p = t - l.cu_seqlens[seg];
    }
  } else {
    p = (int)l.seqlen_div.mod((uint32_t)t);
  }
  return p < 0 ? 0 : (p >= n_pos ? n_pos - 1 : p);
}

__device__ __forceinline__ int rope_position(const TokenLayout &l, int t, int n_pos) {
  int p;
  if (l.position_ids) {
    p = l.position_ids[t];
  } else if (l.cu_seqlens) {
    p = t - l.cu_seqlens[find_segment(l, t)];
  } else {
    p = (int)l.seqlen_div.mod((uint32_t)t);
  }
  return p < 0 ? 0 : (p >= n_pos ? n_pos - 1 : p);
}

}  // namespace muse
