/*
 * libmuseattn -- the Muse Spark Open text-decoder attention core on MI355X (gfx950).
 *
 * The path runs from post-projection Q/K/V and gate logits to the bf16 tensor
 * that feeds o_proj:
 *
 *   Q/K RMSNorm (FP32 accumulation, zero-centred gain) -> bf16
 *   -> query_scale -> adjacent-pair RoPE (FP32 frequencies, FP32 rotation) -> bf16
 *   -> causal GQA softmax attention (BSHD or packed THD, optional sliding window) -> bf16
 *   -> parameter-free output RMSNorm x sigmoid(gate) -> bf16 [tokens, Hq * D]
 *
 * Definitions come from the NeMo AutoModel API reference pages of the
 * muse_spark package: the "layers" page (MuseSparkAttention, MuseSparkRMSNorm,
 * MuseSparkRotaryEmbedding, _rms_norm_core, _qk_norm_rope_core,
 * apply_rotary_embedding, _repeat_kv, _output_norm_gate_core), the "model"
 * page (_causal_mask, _validate_thd_documents, MuseSparkTextModel.forward) and
 * the "vision" page (MuseSparkVisionAttention, _apply_vision_rope,
 * _rope_frequencies).  The backward entry points are the chain rule through
 * the same stages (the pages train the module with autograd).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - bf16 tensors are passed as void pointers to bfloat16 bit patterns in
 *   device memory.  They are token-major and contiguous: Q, gate, O and out
 *   are [N, Hq, D]; K, V and K-hat are [N, Hkv, D] (token stride H*D, head
 *   stride D).  BSHD [B, S, H, D] and packed THD [T, H, D] share this layout:
 *   N = B*S for BSHD and N = T for THD.
 * - float pointers marked "fp32" are device memory.
 * - Alignment: bf16 tensors, gains and cos/sin tables must be 16-byte
 *   aligned (the kernels move them in 16-byte vectors); per-row fp32 outputs
 *   (rstd, lse) and int32 layout arrays 4-byte aligned.  Misaligned pointers
 *   are rejected with MUSE_ERR_INVALID_ARG.
 * - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call
 *   only enqueues work on that stream and returns without synchronising.
 * - The caller owns every buffer, scratch memory included: entry points that
 *   need scratch take a caller workspace (`workspace`, `workspace_bytes`) of
 *   at least the size the matching *_workspace_size query reports for the
 *   same params, layout and current device (0 bytes: NULL is accepted).  A
 *   workspace is 16-byte aligned, needs no initial contents, is overwritten
 *   by the call, and must not overlap any input or output; calls that share
 *   one must not overlap in time (stream order suffices).  The library
 *   allocates no device or pinned memory, keeps no state between calls (a
 *   thread's last error message aside) and is reentrant.  Outputs must not overlap any input or
 *   other output of the same call (the pages return independent tensors);
 *   overlapping ranges are rejected with MUSE_ERR_INVALID_ARG.
 * - Arguments are validated on the host before anything is enqueued.  An
 *   error leaves every output untouched.  muse_last_error() gives a message.
 * - Setting MUSE_DEBUG_VALIDATE=1 in the environment makes calls copy the
 *   device layout arrays to the host -- synchronising the stream, the only
 *   case in which a call waits -- and check them: cu_seqlens with
 *   muse_validate_cu_seqlens, and position_ids (where a RoPE table is read)
 *   against [0, n_pos).  Without it, a malformed cu_seqlens or an
 *   out-of-range position gives unspecified results but every memory access
 *   stays inside the buffers implied by the host-visible sizes.
 */
#ifndef MUSE_ATTN_H
#define MUSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MUSE_OK = 0,
  MUSE_ERR_INVALID_ARG = 1, /* null pointer, bad size, Hq % Hkv != 0, overlap ... */
  MUSE_ERR_UNSUPPORTED = 2, /* valid by the pages, not built here (e.g. D not in {64,128}) */
  MUSE_ERR_DEVICE = 3       /* a HIP call or kernel launch failed */
} muse_status;

/*
 * Per-layer attention parameters (layers page, MuseSparkAttention attributes).
 *
 * head_dim            D; even.  Kernels exist for D = 64 and D = 128.
 * num_heads           Hq, query (and gate/output) heads.
 * num_key_value_heads Hkv; Hq % Hkv == 0.  Query head h reads key/value head
 *                     h / (Hq / Hkv) (KV repeated to the query-head count,
 *                     _repeat_kv).
 * sliding_window      W > 0: query i sees keys j with i - W < j <= i (W keys
 *                     including itself, model page _causal_mask).  W <= 0: no
 *                     window (the pages' None).
 * use_rope            non-zero: rotate Q and K (layers page, layer_uses_rope).
 * upcast_rope         non-zero: FP32 rotation (apply_rotary_embedding upcast=True,
 *                     the original checkpoint's arithmetic).  Zero: rotation in the
 *                     Q/K dtype (upcast=False, the HF release, where each of the
 *                     two products is rounded before the sum): C and S cast to bf16, each
 *                     product rounded to bf16, then the bf16 difference / sum.
 * scaling             softmax scale, head_dim ** -0.5 for this model; finite, > 0.
 * query_scale         multiplier applied after the normalised query's bf16 cast
 *                     (_qk_norm_rope_core), followed by another bf16 cast.  1.0 is a no-op.
 * qk_eps, out_eps     RMSNorm stabilisers added to the mean square (finite, >= 0).
 * gain_center         zero-centred gain offset: effective gain = gain_center + g
 *                     (MuseSparkRMSNorm gain_center, 1.0 by default).
 * bidirectional       non-zero: every key of the query's own row/segment is
 *                     visible, no causal order (vision page,
 *                     MuseSparkVisionAttention: packed bidirectional attention);
 *                     requires sliding_window <= 0.  Zero (the default of a
 *                     zero-initialised struct): causal.
 * skip_qk_norm        non-zero: muse_qk_norm_rope leaves out the RMSNorm and
 *                     gain and only scales/rotates the bf16 Q/K (vision page:
 *                     MuseSparkVisionAttention has no Q/K norm, _apply_vision_rope
 *                     rotates the projected Q/K); gains and rstd outputs must then
 *                     be NULL.  The fused entry points, which normalise the query
 *                     in their prologue, return UNSUPPORTED for it.  Zero: normalise.
 * kv_split            split policy of the attention kernels for grids too small
 *                     to fill the device (a tuning knob, not from the pages): the
 *                     forward and the backward's dQ kernel cut a work item's key
 *                     tiles, the backward's dK/dV kernel a key block's (query
 *                     tile, head) steps, into parts run by separate workgroups
 *                     and summed in part order.
 *                       0  automatic (the default): split only grids with fewer
 *                          work items than resident workgroup slots of the current
 *                          device (two per CU; one for the D = 128 dK/dV kernel),
 *                          into parts of at least 4 steps (at most 4 parts; 8 for
 *                          dK/dV);
 *                       1  never split;
 *                       n >= 2  split every work item of two or more steps into
 *                          min(n, 8) parts (a tuning and testing aid).
 *                     Splitting reorders the sums (results move within rounding);
 *                     a given policy, shape and device always give the same bits,
 *                     fused and unfused alike.  Negative: INVALID_ARG.
 */
typedef struct {
  int32_t head_dim;
  int32_t num_heads;
  int32_t num_key_value_heads;
  int32_t sliding_window;
  int32_t use_rope;
  int32_t upcast_rope;
  float scaling;
  float query_scale;
  float qk_eps;
  float out_eps;
  float gain_center;
  int32_t bidirectional;
  int32_t skip_qk_norm;
  int32_t kv_split;
} muse_attn_params;

/*
 * Token layout (layers page, MuseSparkAttention.forward: qkv_format and
 * cu_seqlens [documents + 1]; model page, _validate_thd_documents).
 *
 * BSHD: cu_seqlens == NULL.  batch >= 0 rows of seqlen >= 0 tokens; each row
 *       is its own causal sequence; N = batch * seqlen.
 * THD:  cu_seqlens != NULL: device int32 [num_segments + 1], non-decreasing,
 *       cu_seqlens[0] == 0, cu_seqlens[num_segments] == total_tokens.  Tokens
 *       attend only inside their own segment.  max_seqlen (host) must be >= the
 *       longest segment; it sizes the launch.  batch and seqlen are ignored.
 * position_ids: optional device int32 [N] RoPE positions (model page, local
 *       position_ids).  NULL means the implicit positions: the index inside the
 *       BSHD row, or inside the THD segment (restarting at 0).  Positions must
 *       lie in [0, n_pos) of the cos/sin table; out-of-range ids are clamped
 *       into it (memory stays safe, the result is unspecified;
 *       MUSE_DEBUG_VALIDATE=1 rejects them with INVALID_ARG).  Masking
 *       always uses the token's index inside its row/segment.
 * attention_mask: optional device uint8 [batch, seqlen] token validity for
 *       BSHD (model page, MuseSparkTextModel.forward attention_mask: nonzero =
 *       valid; a boolean mask's bytes work as is).  A padded key is visible to
 *       no query; the window still counts positions, padded or not; queries
 *       themselves are computed whatever their own validity.  A query left
 *       with no visible key gets the zero row: o = 0, lse = -inf, and the
 *       gated output 0.  Read by the attention entry points only; with THD it
 *       is INVALID_ARG (the pages leave the mask unused for packed THD: pack
 *       the valid tokens instead).
 */
typedef struct {
  int32_t batch;
  int32_t seqlen;
  const int32_t *cu_seqlens;
  int32_t num_segments;
  int32_t total_tokens;
  int32_t max_seqlen;
  const int32_t *position_ids;
  const uint8_t *attention_mask;
} muse_layout;

/*
 * FP32 RoPE cos/sin table (layers page, MuseSparkRotaryEmbedding: FP32
 * adjacent-pair frequencies shared by all text layers; cosine/sine of width
 * head_dim / 2).
 *
 * For position p in [0, n_pos) and pair i in [0, head_dim/2):
 *   inv_i = float(theta ** (-2 i / head_dim))   (evaluated in double, rounded once)
 *   a     = float(p) * inv_i                    (binary32 product)
 *   cos_out[p * head_dim/2 + i] = float(cos(a)), sin_out[...] = float(sin(a))
 *                                               (cos/sin evaluated in double)
 * cos_out, sin_out: device fp32 [n_pos, head_dim/2], written.
 * Errors: INVALID_ARG for theta <= 0 or non-finite, odd or non-positive
 * head_dim, n_pos < 0, null outputs (when n_pos > 0), overlapping outputs.
 */
muse_status muse_rope_cos_sin(float theta, int32_t head_dim, int32_t n_pos, float *cos_out,
                              float *sin_out, void *stream);

/*
 * FP32 2-D RoPE cos/sin table of one row-major patch grid (vision page,
 * _rope_frequencies: adjacent-pair 2-D frequencies [H*W, D/2, 2], read as a
 * cos and a sin table of [H*W, D/2]).
 *
 * Patch p = y * grid_w + x (row y, column x).  With Q = head_dim / 4 and
 * inv_j = float(theta ** (-2 j / (head_dim / 2))) for j in [0, Q) (double,
 * rounded once), pair i of patch p has the angle
 *   a = float(y) * inv_i          for i <  Q   (the row half)
 *   a = float(x) * inv_(i - Q)    for i >= Q   (the column half)
 * (binary32 products), and cos_out[p * head_dim/2 + i] = float(cos(a)),
 * sin_out[...] = float(sin(a)) (double, rounded once): each half is the 1-D
 * table of a head_dim/2-wide head at that coordinate.  Several grids packed
 * into one THD batch use one table each (or one concatenated table) and
 * position_ids that point each patch at its row.
 * cos_out, sin_out: device fp32 [grid_h * grid_w, head_dim/2], written.
 * Errors: INVALID_ARG for theta <= 0 or non-finite, head_dim not a positive
 * multiple of 4, grid_h or grid_w < 0, null outputs (when the grid is not
 * empty), overlapping outputs, more than 2^31 - 1 patches.
 */
muse_status muse_rope_cos_sin_2d(float theta, int32_t head_dim, int32_t grid_h, int32_t grid_w,
                                 float *cos_out, float *sin_out, void *stream);

/*
 * Q/K RMSNorm + gain + bf16 cast + query_scale + adjacent-pair RoPE
 * (layers page, _qk_norm_rope_core, _rms_norm_core, apply_rotary_embedding).
 *
 * For every (token, head) row x of D bf16 values:
 *   r = 1 / sqrt(mean(x^2) + qk_eps)                   (FP32 accumulation)
 *   y = bf16(x * r * (gain_center + g))                 (no gain multiply when g is NULL;
 *                                                        y = x when skip_qk_norm)
 *   Q only: y = bf16(y * query_scale)
 *   use_rope: (y0, y1) of each adjacent pair -> bf16(y0 C - y1 S), bf16(y0 S + y1 C)
 *             in FP32, with C, S = cos/sin[position][pair].
 *
 * q       [N, Hq, D] bf16 in;  q_out [N, Hq, D] bf16 out.   Both NULL: skip Q.
 * k       [N, Hkv, D] bf16 in; k_out [N, Hkv, D] bf16 out.  Both NULL: skip K.
 * q_gain, k_gain  fp32 [D] raw zero-centred gains, or NULL (parameter-free).
 *                 The same pointer may be passed for both (one shared qk_norm).
 * cos, sin        fp32 [n_pos, D/2] table from muse_rope_cos_sin; required
 *                 when use_rope, ignored otherwise.  Implicit positions need
 *                 n_pos >= seqlen (BSHD) or >= max_seqlen (THD).
 * q_rstd, k_rstd  optional fp32 [N, Hq] / [N, Hkv] outputs of r (NULL with skip_qk_norm).
 * Errors: INVALID_ARG (see conventions; also when both q and k are NULL or an
 * input is given without its output), UNSUPPORTED (D not in {64,128}), DEVICE.
 */
muse_status muse_qk_norm_rope(const muse_attn_params *params, const muse_layout *layout,
                              const void *q, const void *k, const float *q_gain,
                              const float *k_gain, const float *cos, const float *sin,
                              int32_t n_pos, void *q_out, void *k_out, float *q_rstd,
                              float *k_rstd, void *stream);

/*
 * muse_qk_norm_rope with the 1-D RoPE table built in the same launch (layers
 * page, MuseSparkRotaryEmbedding and _qk_norm_rope_core): instead of reading
 * cos/sin, the call evaluates the table rows of the positions its tokens have
 * -- every entry exactly as muse_rope_cos_sin(theta, head_dim, n_pos) writes
 * it (same bits) -- rotates with them, and writes those rows into cos_out /
 * sin_out, so that a following muse_attn_fused_fwd (or muse_qk_norm_rope)
 * can read them.  Rows of positions no token has are left untouched; with
 * implicit positions (no position_ids) every position below the longest
 * row/segment is written.  Tokens that share a position write identical bits.
 *
 * theta     as muse_rope_cos_sin.
 * n_pos     rows of cos_out / sin_out (the position rules of muse_qk_norm_rope).
 * cos_out, sin_out  device fp32 [n_pos, D/2], written (rows as above).
 * Other arguments as muse_qk_norm_rope.
 * Errors: as muse_qk_norm_rope; INVALID_ARG also when use_rope is 0, theta is
 * not finite and > 0, or cos_out / sin_out overlap each other or any input.
 */
muse_status muse_qk_norm_rope_table(const muse_attn_params *params, const muse_layout *layout,
                                    const void *q, const void *k, const float *q_gain,
                                    const float *k_gain, float theta, int32_t n_pos,
                                    float *cos_out, float *sin_out, void *q_out, void *k_out,
                                    float *q_rstd, float *k_rstd, void *stream);

/*
 * Causal GQA softmax attention on normalised, rotated Q/K (layers page,
 * MuseSparkAttention: scaling = head_dim ** -0.5, GQA groups, sliding_window;
 * model page, _causal_mask).
 *
 * For every query token i (index inside its row/segment) and head h, with
 * kv = h / (Hq / Hkv) and J(i) the visible keys (j <= i, j > i - W when W > 0,
 * same row/segment; every key of the row/segment when bidirectional; padded
 * keys of layout->attention_mask removed):
 *   s_j = scaling * <q_hat[i,h], k_hat[j,kv]>   (bf16 products, FP32 accumulation)
 *   o[i,h] = bf16( sum_j softmax(s)_j v[j,kv] ),  lse[i,h] = ln sum_j exp(s_j)
 *
 * q_hat [N, Hq, D], k_hat [N, Hkv, D], v [N, Hkv, D]: bf16 in.
 * o     [N, Hq, D] bf16 out.  lse: optional fp32 [N, Hq] out (natural log).
 *
 * Small grids split each work item's keys into parts (params->kv_split)
 * whose partial results go through the workspace: workspace_bytes >=
 * muse_attn_fwd_workspace_size(params, layout) (0 when the call does not
 * split; then workspace may be NULL).  The partial slots need no initial
 * contents; the call zeroes its arrival counters on the stream first.
 * Errors: INVALID_ARG (also a missing, misaligned or too small workspace),
 * UNSUPPORTED (D not in {64,128}), DEVICE.
 */
muse_status muse_gqa_attn_fwd(const muse_attn_params *params, const muse_layout *layout,
                              const void *q_hat, const void *k_hat, const void *v, void *o,
                              float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Workspace bytes the attention forward (muse_gqa_attn_fwd,
 * muse_attn_fused_fwd, muse_attn_core_fwd) needs for params and layout on
 * the current device: the KV-split partial slots and arrival counters, 0 when
 * the split policy leaves the grid whole.
 * Errors: as the parameter and layout checks of muse_gqa_attn_fwd; INVALID_ARG
 * for a NULL bytes.
 */
muse_status muse_attn_fwd_workspace_size(const muse_attn_params *params, const muse_layout *layout,
                                         size_t *bytes);

/*
 * Parameter-free output RMSNorm times the sigmoid output gate (layers page,
 * _output_norm_gate_core).
 *
 * For every (token, head) row o of D bf16 values and its gate row:
 *   r = 1 / sqrt(mean(o^2) + out_eps)                   (FP32)
 *   out = bf16( o * r * 1 / (1 + exp(-gate)) )         (FP32, one final cast)
 *
 * o, gate [N, Hq, D] bf16 in; out [N, Hq, D] bf16 out (= [N, Hq*D], o_proj's input).
 * o_rstd: optional fp32 [N, Hq] out.
 * Errors: INVALID_ARG, UNSUPPORTED (D not in {64,128}), DEVICE.
 */
muse_status muse_out_norm_gate(const muse_attn_params *params, const muse_layout *layout,
                               const void *o, const void *gate, void *out, float *o_rstd,
                               void *stream);

/*
 * The whole core in one call: muse_qk_norm_rope -> muse_gqa_attn_fwd ->
 * muse_out_norm_gate, with the query norm/RoPE fused into the attention
 * kernel's Q load and the output norm and gate applied to the attention
 * result in registers.  Results equal the three-call chain.
 *
 * q, gate [N, Hq, D]; k, v [N, Hkv, D]: bf16 in.  q_gain, k_gain, cos, sin,
 * n_pos as in muse_qk_norm_rope.
 * k_hat_out [N, Hkv, D] bf16 out: the normalised, rotated keys (what a KV cache
 *           keeps).  Required: the attention reads it back.
 * out       [N, Hq, D] bf16 out.   lse: optional fp32 [N, Hq] out.
 * workspace, workspace_bytes: as muse_gqa_attn_fwd (muse_attn_fwd_workspace_size).
 * Errors: as the three calls above.
 */
muse_status muse_attn_core_fwd(const muse_attn_params *params, const muse_layout *layout,
                               const void *q, const void *k, const void *v, const void *gate,
                               const float *q_gain, const float *k_gain, const float *cos,
                               const float *sin, int32_t n_pos, void *k_hat_out, void *out,
                               float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The attention kernel of muse_attn_core_fwd on its own: the query norm/RoPE
 * prologue and the output norm/gate epilogue fused, keys already normalised
 * and rotated (by muse_qk_norm_rope, or held that way in a key cache).
 * muse_attn_core_fwd is muse_qk_norm_rope on K followed by this call.
 *
 * q, gate [N, Hq, D]; k_hat, v [N, Hkv, D]: bf16 in.  q_gain, cos, sin, n_pos
 * as in muse_qk_norm_rope (Q side).  out [N, Hq, D] bf16 out; lse optional
 * fp32 [N, Hq] out.  workspace, workspace_bytes: as muse_gqa_attn_fwd.
 * Errors: as muse_gqa_attn_fwd, plus the table rules of muse_qk_norm_rope.
 */
muse_status muse_attn_fused_fwd(const muse_attn_params *params, const muse_layout *layout,
                                const void *q, const void *k_hat, const void *v, const void *gate,
                                const float *q_gain, const float *cos, const float *sin,
                                int32_t n_pos, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * ---------------------------------------------------------------- backward
 *
 * The gradients of the forward stages above, each following autograd's
 * dtypes: a gradient of a bf16 tensor is bf16, gain gradients are fp32.
 * The rotation's backward is its transpose: by the FP32 cos/sin, or, after
 * the Q/K-dtype rotation (upcast_rope = 0), by their bf16 casts (the bf16
 * roundings of its products and sums differentiated as the identity).
 * Entry points that
 * need scratch memory take a caller-owned workspace (see the conventions).
 * Results are deterministic: fixed reduction orders (a split's arrival
 * counters only pick which part sums the others, in part order).
 */

/*
 * Backward of the output norm + gate (layers page, _output_norm_gate_core).
 * With y = o r, r = 1 / sqrt(mean(o^2) + out_eps), s = sigmoid(gate):
 *   dgate = bf16(dout y s (1 - s)),  d_o = bf16(r dout s - r^3 o mean(dout s o)),
 *   delta = sum_d d_o * o  (fp32, the softmax correction of muse_gqa_attn_bwd).
 * o, gate, dout [N, Hq, D] bf16 in; d_o, dgate [N, Hq, D] bf16 out; delta fp32 [N, Hq] out.
 * Errors: INVALID_ARG, UNSUPPORTED (D not in {64,128}), DEVICE.
 */
muse_status muse_out_norm_gate_bwd(const muse_attn_params *params, const muse_layout *layout,
                                   const void *o, const void *gate, const void *dout, void *d_o,
                                   void *dgate, float *delta, void *stream);

/*
 * delta = sum_d d_o * o (fp32 [N, Hq]) for an attention backward without the
 * output gate (o, d_o [N, Hq, D] bf16).
 */
muse_status muse_attn_bwd_delta(const muse_attn_params *params, const muse_layout *layout,
                                const void *o, const void *d_o, float *delta, void *stream);

/*
 * Backward of muse_gqa_attn_fwd (same masking rules: causal/window,
 * bidirectional, padded keys).  With P the softmax of the forward,
 * recomputed as exp(scaling q_hat k_hat^T - lse):
 *   dP = d_o v^T,  dS = P (dP - delta),
 *   dq_hat = bf16(scaling dS k_hat),  dk_hat = bf16(scaling sum_heads dS^T q_hat),
 *   dv = bf16(sum_heads P^T d_o)   (sums over the query heads of each KV head).
 * q_hat [N, Hq, D], k_hat, v [N, Hkv, D], d_o [N, Hq, D] bf16 in; lse (natural
 * log, from the forward) and delta fp32 [N, Hq] in; dq_hat [N, Hq, D], dk_hat,
 * dv [N, Hkv, D] bf16 out.  A padded key gets zero gradients.
 * workspace: muse_gqa_attn_bwd_workspace_size bytes (the split's partial sums
 * and arrival counters; 0 when params->kv_split leaves both kernels whole).
 * Errors: INVALID_ARG, UNSUPPORTED (D not in {64,128}), DEVICE.
 */
muse_status muse_gqa_attn_bwd(const muse_attn_params *params, const muse_layout *layout,
                              const void *q_hat, const void *k_hat, const void *v, const void *d_o,
                              const float *lse, const float *delta, void *dq_hat, void *dk_hat,
                              void *dv, void *workspace, size_t workspace_bytes, void *stream);
muse_status muse_gqa_attn_bwd_workspace_size(const muse_attn_params *params,
                                             const muse_layout *layout, size_t *bytes);

/*
 * Backward of muse_qk_norm_rope.  For each row: g = the FP32 inverse rotation
 * of the incoming gradient, (g0 C + g1 S, -g0 S + g1 C), rounded to bf16
 * (C, S = bf16(cos), bf16(sin) when upcast_rope = 0);
 * for Q, g = bf16(g * query_scale); then with x the raw input, r its rstd and
 * w = gain_center + gain (1 without a gain), u = g w:
 *   dx = bf16(r u - r^3 x mean(u x)),  dgain += g x r  (summed over all rows, fp32).
 * skip_qk_norm: dx = g, no gain gradients.
 * q, dq_hat, dq [N, Hq, D] (all three NULL: skip Q); k, dk_hat, dk [N, Hkv, D]
 * (all NULL: skip K); q_gain, k_gain as in the forward; dq_gain, dk_gain fp32
 * [D] out, given exactly when the matching gain is (for one gain shared by
 * Q and K, its gradient is dq_gain + dk_gain); cos/sin as in the forward.
 * workspace: muse_qk_norm_rope_bwd_workspace_size bytes (gain partial sums).
 * Errors: INVALID_ARG, UNSUPPORTED (D not in {64,128}), DEVICE.
 */
muse_status muse_qk_norm_rope_bwd(const muse_attn_params *params, const muse_layout *layout,
                                  const void *q, const void *k, const float *q_gain,
                                  const float *k_gain, const float *cos, const float *sin,
                                  int32_t n_pos, const void *dq_hat, const void *dk_hat, void *dq,
                                  void *dk, float *dq_gain, float *dk_gain, void *workspace,
                                  size_t workspace_bytes, void *stream);
muse_status muse_qk_norm_rope_bwd_workspace_size(const muse_attn_params *params,
                                                 const muse_layout *layout, size_t *bytes);

/*
 * muse_qk_norm_rope_bwd without a workspace, for callers that cannot
 * allocate (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  The gain-gradient partial sums go to scratch memory
 * the library holds in device memory instead: one static array per GPU of
 * 2 x 2048 x 128 floats (2 MiB), held from the first call on that GPU until
 * the process ends.  Every shape muse_qk_norm_rope_bwd accepts fits it; a
 * shape whose partial sums did not fit would get INVALID_ARG.  The call
 * allocates nothing.  All calls on one GPU share its array: calls that
 * overlap in time on one GPU (other streams, other threads, a graph replayed
 * beside another call) race and give wrong gain gradients.  Nothing in the
 * array needs to start at zero (each call overwrites the partial rows it
 * reads).  Arguments, results and errors otherwise as muse_qk_norm_rope_bwd.
 */
muse_status muse_qk_norm_rope_bwd_static(const muse_attn_params *params, const muse_layout *layout,
                                         const void *q, const void *k, const float *q_gain,
                                         const float *k_gain, const float *cos, const float *sin,
                                         int32_t n_pos, const void *dq_hat, const void *dk_hat,
                                         void *dq, void *dk, float *dq_gain, float *dk_gain,
                                         void *stream);

/*
 * Backward of the whole core (muse_attn_core_fwd): gradients of q, k, v, the
 * gate logits and the two gains, from dout [N, Hq, D] bf16.
 * o: the forward's attention output before the output norm ([N, Hq, D] bf16,
 * as muse_gqa_attn_fwd writes it) and lse (fp32 [N, Hq]); both NULL: they are
 * recomputed here (the fused forward keeps neither).  Steps: Q/K norm + RoPE
 * forward into the workspace, muse_out_norm_gate_bwd, muse_gqa_attn_bwd,
 * muse_qk_norm_rope_bwd.
 * Outputs: dq [N, Hq, D], dk, dv [N, Hkv, D], dgate [N, Hq, D] bf16;
 * dq_gain, dk_gain fp32 [D] (given exactly when the matching gain is).
 * workspace: muse_attn_core_bwd_workspace_size bytes.
 * Errors: INVALID_ARG, UNSUPPORTED (D not in {64,128}, skip_qk_norm), DEVICE.
 */
muse_status muse_attn_core_bwd(const muse_attn_params *params, const muse_layout *layout,
                               const void *q, const void *k, const void *v, const void *gate,
                               const float *q_gain, const float *k_gain, const float *cos,
                               const float *sin, int32_t n_pos, const void *o, const float *lse,
                               const void *dout, void *dq, void *dk, void *dv, void *dgate,
                               float *dq_gain, float *dk_gain, void *workspace,
                               size_t workspace_bytes, void *stream);
muse_status muse_attn_core_bwd_workspace_size(const muse_attn_params *params,
                                              const muse_layout *layout, size_t *bytes);

/*
 * Pure host check of a packed layout (model page, _validate_thd_documents):
 * cu_seqlens (host int32 [num_segments + 1]) starts at 0, never decreases,
 * ends at total_tokens, and no segment is longer than max_seqlen.
 * Returns MUSE_OK or MUSE_ERR_INVALID_ARG.  Touches no GPU.
 */
muse_status muse_validate_cu_seqlens(const int32_t *cu_seqlens_host, int32_t num_segments,
                                     int32_t total_tokens, int32_t max_seqlen);

/* Static name of a status code. */
const char *muse_status_string(muse_status status);

/* Message describing the last error returned on the calling thread ("" if none). */
const char *muse_last_error(void);

/* Library version, "major.minor.patch". */
const char *muse_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUSE_ATTN_H */
