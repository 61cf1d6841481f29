"""Plain FP64 CPU oracle for the Muse Spark Open text-decoder attention core.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
helpers with the HIP library and does not import it.

What it computes is defined by the NeMo AutoModel API reference pages for the
``muse_spark`` model package.  Citations name a page and the section on it:

* "layers page" -- ``nemo_automodel.components.models.muse_spark.layers``
  (sections ``MuseSparkAttention``, ``MuseSparkRMSNorm``,
  ``MuseSparkRotaryEmbedding``, ``_rms_norm_core``, ``_qk_norm_rope_core``,
  ``apply_rotary_embedding``, ``_repeat_kv``, ``_output_norm_gate_core``);
* "model page" -- ``nemo_automodel.components.models.muse_spark.model``
  (sections ``_causal_mask`` and ``MuseSparkTextModel.forward``'s
  ``attention_mask``: token validity [batch, sequence]);
* "adapter page" -- ``nemo_automodel.components.models.muse_spark.hf_state_dict_adapter``
  (section ``_permute_rope_rows``);
* "vision page" -- ``nemo_automodel.components.models.muse_spark.vision``
  (sections ``MuseSparkVisionAttention``: packed bidirectional attention;
  ``_apply_vision_rope``, ``_rope_frequencies``: adjacent-pair 2-D RoPE).

The method is a composition of exact definitions (no approximation, heuristic
or iteration), so every function below is that definition written out in
float64, with each dtype boundary the pages name emulated by an explicit
round-to-nearest-even.  Flash-style blocking reaches the plain softmax result
up to rounding order, so attention here is the plain masked softmax.

Readings taken where the pages are silent:
RMS over the last dim per (token, head); eps inside the square root; effective
gain ``f32(gain_center + g)`` applied after normalisation and before the cast;
RoFormer rotation sign with frequencies ``theta**(-2i/D)``; cos/sin of width
D/2; window ``W`` = number of visible causal keys including the query itself;
no attention across packed segments (bidirectional mode: every key of the
query's own segment, no window); a padded key (attention_mask [B,S] False)
is visible to no query, and a query left with no visible key gives the zero
row with lse = -inf; bf16 boundary on the attention output;
sigmoid and output norm in full precision with one final cast; the vision
2-D table gives the first half of the pairs the patch row and the second
half the patch column; the backward (written from the chain rule of these
definitions) takes the delta of the softmax correction from the stored bf16
output, and differentiates the Q/K-dtype rotation as the transpose of the
rotation by its bf16 cos/sin (its bf16 roundings as the identity).

Every function here is pinned by ``tests/test_oracle_pins.py`` and
``tests/test_oracle_bwd_pins.py`` against closed forms, library routines,
torch autograd of an independent float64 forward, finite differences or
brute force; none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "round_bf16",
    "round_f32",
    "rope_inv_freq",
    "rope_cos_sin",
    "rope_cos_sin_2d",
    "rms_normalize",
    "rms_norm",
    "rope_rotate",
    "qk_norm_rope",
    "visible_mask",
    "attention",
    "attention_rows",
    "attention_rows_grouped",
    "out_norm_gate",
    "Segments",
    "attn_core",
    "attn_core_rows",
    "out_norm_gate_bwd",
    "attention_bwd",
    "rope_rotate_bwd",
    "rms_norm_bwd",
    "qk_norm_rope_bwd",
    "attn_core_bwd",
    "attention_bwd_rows",
    "attention_bwd_keys",
]


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bfloat16 bit patterns (uint16)."""
    u32 = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to bfloat16, ties to even, in one step.

    bfloat16 keeps 8 significant bits and the binary32 exponent range; below
    2**-126 the quantum is fixed at 2**-133 (subnormals).  The rounding is done
    directly from float64 so no double rounding through binary32 occurs.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)                       # xf = m * 2**e, 0.5 <= |m| < 1
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(xf / q) * q                   # np.rint rounds half to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
    out[fin] = r
    return out


def round_f32(x) -> np.ndarray:
    """Round float64 values to binary32 (numpy's cast rounds to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Rotary table -- layers page, MuseSparkRotaryEmbedding (one set of FP32
# adjacent-pair frequencies serves every text layer; forward returns cosine and
# sine of shape [batch, sequence, head_dim / 2]).
# --------------------------------------------------------------------------

def rope_inv_freq(theta: float, head_dim: int) -> np.ndarray:
    """FP32 inverse frequencies inv_i = theta**(-2i/D), i < D/2, rounded once."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return round_f32(np.power(np.float64(theta), -2.0 * i / head_dim))


def rope_cos_sin(theta: float, head_dim: int, positions) -> tuple[np.ndarray, np.ndarray]:
    """cos/sin [len(positions), D/2]: FP32 angle p*inv_i, then FP32 cos and sin.

    The angle is the binary32 product of the (exact) position and the FP32
    frequency; its cosine and sine are evaluated in float64 and rounded once.
    """
    p = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    ang = round_f32(p * rope_inv_freq(theta, head_dim)[None, :])
    return round_f32(np.cos(ang)), round_f32(np.sin(ang))


def rope_cos_sin_2d(theta: float, head_dim: int, grid_h: int, grid_w: int):
    """cos/sin [grid_h*grid_w, D/2] of one row-major patch grid (vision page,
    _rope_frequencies: adjacent-pair 2-D frequencies [H*W, D/2, 2]).

    Reading (the page gives only the shape): the trailing 2 is (cos, sin);
    patch p = y*grid_w + x; the first D/4 pairs rotate with the row y and the
    last D/4 with the column x, each half at the 1-D frequencies of a
    D/2-wide head, theta**(-2j/(D/2)).  The angle is a binary32 product and
    cos/sin are rounded once, as in the 1-D table.
    """
    if head_dim % 4:
        raise ValueError("2-D RoPE needs head_dim % 4 == 0")
    quarter = head_dim // 4
    j = np.arange(quarter, dtype=np.float64)
    inv = round_f32(np.power(np.float64(theta), -2.0 * j / (head_dim // 2)))
    y = np.repeat(np.arange(grid_h, dtype=np.float64), grid_w)[:, None]
    x = np.tile(np.arange(grid_w, dtype=np.float64), grid_h)[:, None]
    ang = np.concatenate([round_f32(y * inv[None, :]), round_f32(x * inv[None, :])], axis=1)
    return round_f32(np.cos(ang)), round_f32(np.sin(ang))


# --------------------------------------------------------------------------
# RMSNorm -- layers page, MuseSparkRMSNorm / effective_weight / _rms_norm_core
# (normalisation in FP32, the effective gain applied before the cast to the
# output dtype; eps is added to the mean of the squares).
# --------------------------------------------------------------------------

def rms_normalize(x: np.ndarray, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """Unrounded x / sqrt(mean(x**2) + eps) over the last dim, and that rstd."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(ms + float(round_f32(eps)))
    return x * rstd, rstd[..., 0]


def rms_norm(x: np.ndarray, eps: float, gain=None, gain_center: float = 1.0):
    """bf16(normalize(x) * w) with w = f32(gain_center + g); no gain when None.

    Returns (bf16-valued float64 array, rstd float64 [...]).
    """
    y, rstd = rms_normalize(x, eps)
    if gain is not None:
        w = round_f32(np.float64(round_f32(gain_center)) + np.asarray(gain, dtype=np.float64))
        y = y * w
    return round_bf16(y), rstd


# --------------------------------------------------------------------------
# RoPE rotation -- layers page, apply_rotary_embedding (pairs of adjacent
# elements; the original checkpoint computes the rotation in FP32, upcast=True).
# --------------------------------------------------------------------------

def rope_rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, upcast: bool = True) -> np.ndarray:
    """Rotate each adjacent pair (x_{2i}, x_{2i+1}) by its angle.

    ``cos``/``sin`` broadcast against x[..., 0::2].  The rotation is
    (x0*C - x1*S, x0*S + x1*C), RoFormer's 2-D rotation block.

    upcast=True (the original checkpoint, layers page apply_rotary_embedding):
    the rotation in full precision, one bf16 cast.  upcast=False (the HF
    release, same section: both products rounded in the Q/K dtype before they
    are added): C and S cast to bf16, each product rounded to bf16, then the
    bf16 sum or difference -- every step a bf16 operation.
    """
    x = np.asarray(x, dtype=np.float64)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty_like(x)
    if upcast:
        y[..., 0::2] = round_bf16(x0 * cos - x1 * sin)
        y[..., 1::2] = round_bf16(x0 * sin + x1 * cos)
    else:
        c = round_bf16(np.asarray(cos, dtype=np.float64))
        s = round_bf16(np.asarray(sin, dtype=np.float64))
        y[..., 0::2] = round_bf16(round_bf16(x0 * c) - round_bf16(x1 * s))
        y[..., 1::2] = round_bf16(round_bf16(x0 * s) + round_bf16(x1 * c))
    return y


# --------------------------------------------------------------------------
# Sequences: BSHD rows or packed THD segments (layers page, MuseSparkAttention
# .forward: cu_seqlens [documents + 1]; model page, position_ids are local).
# --------------------------------------------------------------------------

class Segments:
    """Token ranges [start, start+len) that attend only within themselves."""

    def __init__(self, starts, lengths):
        self.starts = [int(s) for s in starts]
        self.lengths = [int(n) for n in lengths]

    @classmethod
    def bshd(cls, batch: int, seqlen: int) -> "Segments":
        return cls([b * seqlen for b in range(batch)], [seqlen] * batch)

    @classmethod
    def thd(cls, cu_seqlens) -> "Segments":
        cu = [int(c) for c in cu_seqlens]
        return cls(cu[:-1], [cu[i + 1] - cu[i] for i in range(len(cu) - 1)])

    @property
    def total(self) -> int:
        return sum(self.lengths)

    def local_positions(self) -> np.ndarray:
        """Position of each token inside its own sequence/segment (restarting at 0)."""
        end = max((s + n for s, n in zip(self.starts, self.lengths)), default=0)
        pos = np.zeros(end, dtype=np.int64)
        for s, n in zip(self.starts, self.lengths):
            pos[s:s + n] = np.arange(n)
        return pos

    def locate(self, token: int) -> tuple[int, int]:
        """(segment start, segment length) of the segment holding ``token``."""
        for s, n in zip(self.starts, self.lengths):
            if s <= token < s + n:
                return s, n
        raise IndexError(token)


# --------------------------------------------------------------------------
# Q/K norm + query scale + RoPE -- layers page, _qk_norm_rope_core
# (the query scale multiplies the normalised query after its dtype cast).
# --------------------------------------------------------------------------

def qk_norm_rope(q, k, *, eps, q_gain=None, k_gain=None, gain_center=1.0,
                 query_scale=1.0, use_rope=True, cos=None, sin=None, upcast_rope=True,
                 normalize=True):
    """Q [N,Hq,D], K [N,Hkv,D] -> (q_hat, k_hat, q_rstd [N,Hq], k_rstd [N,Hkv]).

    ``cos``/``sin`` are the per-token rows [N, D/2] (already indexed by each
    token's position); they are ignored when ``use_rope`` is false.
    normalize=False is the vision attention's rotation (vision page,
    MuseSparkVisionAttention has no Q/K norm; _apply_vision_rope rotates the
    bf16 projections directly): no RMSNorm, no gain, rstd returned as None.
    """
    if normalize:
        q1, q_rstd = rms_norm(q, eps, q_gain, gain_center)
        k1, k_rstd = rms_norm(k, eps, k_gain, gain_center)
    else:
        q1, k1, q_rstd, k_rstd = np.asarray(q, np.float64), np.asarray(k, np.float64), None, None
    q1 = round_bf16(q1 * np.float64(round_f32(query_scale)))
    if use_rope:
        c = np.asarray(cos, dtype=np.float64)[:, None, :]
        s = np.asarray(sin, dtype=np.float64)[:, None, :]
        q1 = rope_rotate(q1, c, s, upcast_rope)
        k1 = rope_rotate(k1, c, s, upcast_rope)
    return q1, k1, q_rstd, k_rstd


# --------------------------------------------------------------------------
# Attention -- layers page, MuseSparkAttention (scaling = head_dim**-0.5,
# num_key_value_groups = num_heads // num_key_value_heads), _repeat_kv
# (KV heads repeated to the query-head count); model page, _causal_mask
# (the window W counts the causal key positions one query sees).
# --------------------------------------------------------------------------

def visible_mask(qpos: np.ndarray, kpos: np.ndarray, window: int, causal: bool = True,
                 key_ok=None) -> np.ndarray:
    """Key j visible to query i iff j <= i and, with a window W > 0, j > i - W.

    causal=False is the packed bidirectional attention of the vision tower
    (vision page, MuseSparkVisionAttention): every key of the segment is
    visible (no window).  ``key_ok`` (bool per key) is the token-validity
    mask of a padded batch (model page, _causal_mask with an attention_mask
    [B,S], True = valid): a padded key is visible to no query; the window
    still counts positions."""
    i = np.asarray(qpos)[:, None]
    j = np.asarray(kpos)[None, :]
    if not causal:
        vis = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    else:
        vis = j <= i
        if window and window > 0:
            vis &= j > i - window
    if key_ok is not None:
        vis &= np.asarray(key_ok, dtype=bool)[None, :]
    return vis


def _attend_block(qb, kseg, vseg, qpos, window, scaling, causal=True, key_ok=None):
    """Softmax attention of query rows qb [m,D] over one segment's keys [L,D].

    A row with no visible key (possible only with padded keys) is the zero
    row with lse = -inf."""
    s = float(scaling) * (qb @ kseg.T)
    vis = visible_mask(qpos, np.arange(kseg.shape[0]), window, causal, key_ok)
    seen = vis.any(axis=1)
    s = np.where(vis, s, -np.inf)
    mx = np.where(seen, s.max(axis=1, initial=-np.inf), 0.0)[:, None]
    e = np.where(vis, np.exp(s - mx), 0.0)
    z = e.sum(axis=1, keepdims=True)
    o = np.where(seen[:, None], (e @ vseg) / np.where(z > 0, z, 1.0), 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(seen, mx[:, 0] + np.log(np.where(seen, z[:, 0], 1.0)), -np.inf)
    return o, lse


def attention(q_hat, k_hat, v, segments: Segments, *, window=0, scaling, row_block=2048, causal=True,
              key_valid=None):
    """Exact causal (or, causal=False, bidirectional) GQA softmax attention.
    Returns (bf16(o) [N,Hq,D], lse [N,Hq]).

    Query head h reads key/value head h // (Hq // Hkv).  lse uses the natural
    log.  Rows outside every segment are left at zero.  ``key_valid`` [N]
    (bool, per token) masks padded keys; a query left with no visible key
    gets the zero row and lse = -inf.
    """
    q_hat = np.asarray(q_hat, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q_hat.shape
    hkv = k_hat.shape[1]
    groups = hq // hkv
    o = np.zeros_like(q_hat)
    lse = np.zeros((n, hq))
    for s0, length in zip(segments.starts, segments.lengths):
        for h in range(hq):
            g = h // groups
            kseg = k_hat[s0:s0 + length, g]
            vseg = v[s0:s0 + length, g]
            kok = None if key_valid is None else np.asarray(key_valid)[s0:s0 + length]
            for r0 in range(0, length, row_block):
                r1 = min(length, r0 + row_block)
                ob, lb = _attend_block(q_hat[s0 + r0:s0 + r1, h], kseg, vseg,
                                       np.arange(r0, r1), window, scaling, causal, kok)
                o[s0 + r0:s0 + r1, h] = ob
                lse[s0 + r0:s0 + r1, h] = lb
    return round_bf16(o), lse


def attention_rows(q_hat_rows, k_hat, v, segments: Segments, rows, *, num_heads, window=0, scaling,
                   causal=True, key_valid=None):
    """Attention for selected (token, head) rows only.

    ``q_hat_rows`` [len(rows), D] holds the normalised/rotated query of each
    selected row.  Returns (bf16(o) [len(rows), D], lse [len(rows)]).
    """
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    groups = num_heads // k_hat.shape[1]
    o = np.zeros((len(rows), k_hat.shape[2]))
    lse = np.zeros(len(rows))
    for r, (t, h) in enumerate(rows):
        s0, length = segments.locate(int(t))
        g = int(h) // groups
        kok = None if key_valid is None else np.asarray(key_valid)[s0:s0 + length]
        ob, lb = _attend_block(np.asarray(q_hat_rows[r], dtype=np.float64)[None, :],
                               k_hat[s0:s0 + length, g], v[s0:s0 + length, g],
                               np.array([int(t) - s0]), window, scaling, causal, kok)
        o[r] = ob[0]
        lse[r] = lb[0]
    return round_bf16(o), lse


def attention_rows_grouped(q_hat_rows, k_hat, v, segments: Segments, rows, *, num_heads, window=0, scaling,
                           causal=True, key_valid=None, block=64):
    """attention_rows for many rows at once: the same masked softmax of each
    selected (token, head) row over its segment's keys (layers page,
    MuseSparkAttention; model page, _causal_mask), evaluated for up to
    ``block`` rows of one (segment, KV head) together.  A block's keys are the
    run of its segment that holds every key some row of the block sees (for
    causal rows: from the earliest window start to the latest query); keys
    outside a row's visible set get probability zero exactly, as in the plain
    definition.  Returns (bf16(o) [len(rows), D], lse [len(rows)])."""
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    groups = num_heads // k_hat.shape[1]
    o = np.zeros((len(rows), k_hat.shape[2]))
    lse = np.zeros(len(rows))
    by_unit = {}
    for r, (t, h) in enumerate(rows):
        s0, length = segments.locate(int(t))
        by_unit.setdefault((s0, length, int(h) // groups), []).append(r)
    for (s0, length, g), idx in by_unit.items():
        idx.sort(key=lambda r: int(rows[r][0]))
        kok_seg = None if key_valid is None else np.asarray(key_valid)[s0:s0 + length]
        for b0 in range(0, len(idx), block):
            sel = idx[b0:b0 + block]
            qpos = np.array([int(rows[r][0]) - s0 for r in sel])
            if causal:
                lo = max(0, int(qpos.min()) - window + 1) if window and window > 0 else 0
                hi = int(qpos.max()) + 1
            else:
                lo, hi = 0, length
            qb = np.stack([np.asarray(q_hat_rows[r], dtype=np.float64) for r in sel])
            kok = None if kok_seg is None else kok_seg[lo:hi]
            # positions shifted by lo: visibility depends only on differences
            ob, lb = _attend_block(qb, k_hat[s0 + lo:s0 + hi, g], v[s0 + lo:s0 + hi, g], qpos - lo, window,
                                   scaling, causal, kok)
            o[sel] = ob
            lse[sel] = lb
    return round_bf16(o), lse


# --------------------------------------------------------------------------
# Output norm and gate -- layers page, _output_norm_gate_core (parameter-free
# output RMSNorm, sigmoid gate with the output's shape, gated output in the
# original dtype).
# --------------------------------------------------------------------------

def out_norm_gate(o, gate, eps):
    """bf16(rmsnorm(o) * sigmoid(gate)), both in full precision; returns (out, rstd)."""
    y, rstd = rms_normalize(o, eps)
    g = np.asarray(gate, dtype=np.float64)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    return round_bf16(y * sig), rstd


# --------------------------------------------------------------------------
# The whole core -- layers page, MuseSparkAttention.forward: Q/K norm + RoPE
# (_qk_norm_rope_core), attention, then _output_norm_gate_core, ending in the
# tensor fed to o_proj.
# --------------------------------------------------------------------------

def attn_core(q, k, v, gate, segments: Segments, *, theta, eps, out_eps, scaling,
              window=0, use_rope=True, q_gain=None, k_gain=None, gain_center=1.0,
              query_scale=1.0, position_ids=None, upcast_rope=True, causal=True, key_valid=None):
    """Full forward over every row.  Inputs are float64 arrays of bf16 values.

    Returns a dict with q_hat, k_hat, q_rstd, k_rstd, o (bf16 values), lse,
    o_rstd and out (bf16 values [N,Hq,D]).
    """
    d = q.shape[-1]
    pos = segments.local_positions() if position_ids is None else np.asarray(position_ids)
    cos, sin = rope_cos_sin(theta, d, pos) if use_rope else (None, None)
    q_hat, k_hat, q_rstd, k_rstd = qk_norm_rope(
        q, k, eps=eps, q_gain=q_gain, k_gain=k_gain, gain_center=gain_center,
        query_scale=query_scale, use_rope=use_rope, cos=cos, sin=sin, upcast_rope=upcast_rope)
    o, lse = attention(q_hat, k_hat, v, segments, window=window, scaling=scaling, causal=causal,
                       key_valid=key_valid)
    out, o_rstd = out_norm_gate(o, gate, out_eps)
    return dict(q_hat=q_hat, k_hat=k_hat, q_rstd=q_rstd, k_rstd=k_rstd, o=o, lse=lse,
                o_rstd=o_rstd, out=out)


def attn_core_rows(q_rows, k, v, gate_rows, segments: Segments, rows, *, num_heads, theta, eps,
                   out_eps, scaling, window=0, use_rope=True, q_gain=None, k_gain=None, gain_center=1.0,
                   query_scale=1.0, position_ids=None, upcast_rope=True, causal=True, key_valid=None,
                   grouped=False):
    """The full forward for selected (token, head) rows only.

    ``q_rows``/``gate_rows`` [R, D] hold the query and gate values of the R
    selected rows (``num_heads`` query heads in all); K and V [N, Hkv, D] are
    used whole.  Returns a dict with
    q_hat [R,D], k_hat [N,Hkv,D], o [R,D], lse [R], o_rstd [R] and out [R,D].
    """
    rows = [(int(t), int(h)) for t, h in rows]
    d = k.shape[-1]
    pos = segments.local_positions() if position_ids is None else np.asarray(position_ids)
    tok = np.array([t for t, _ in rows], dtype=np.int64)
    if use_rope:
        kc, ks = rope_cos_sin(theta, d, pos)
        qc, qs = kc[tok], ks[tok]
    else:
        kc = ks = qc = qs = None
    q_hat = _q_rows(np.asarray(q_rows, dtype=np.float64), eps, q_gain, gain_center, query_scale,
                    use_rope, qc, qs, upcast_rope)
    k1, _ = rms_norm(k, eps, k_gain, gain_center)
    k_hat = rope_rotate(k1, kc[:, None, :], ks[:, None, :], upcast_rope) if use_rope else k1
    attend = attention_rows_grouped if grouped else attention_rows
    o, lse = attend(q_hat, k_hat, v, segments, rows, num_heads=num_heads, window=window, scaling=scaling,
                    causal=causal, key_valid=key_valid)
    out, o_rstd = out_norm_gate(o, np.asarray(gate_rows, dtype=np.float64), out_eps)
    return dict(q_hat=q_hat, k_hat=k_hat, o=o, lse=lse, o_rstd=o_rstd, out=out)


def _q_rows(q_sel, eps, q_gain, gain_center, query_scale, use_rope, cos, sin, upcast_rope=True):
    q1, _ = rms_norm(q_sel, eps, q_gain, gain_center)
    q1 = round_bf16(q1 * np.float64(round_f32(query_scale)))
    if use_rope:
        q1 = rope_rotate(q1, cos, sin, upcast_rope)
    return q1


# --------------------------------------------------------------------------
# Backward of the core.  The pages train this module with autograd (layers
# page, MuseSparkDecoderLayer is a GradientCheckpointingLayer; the compiled
# cores and SDPA/TE are differentiated by their frameworks), so the backward
# is the chain rule through the forward above, stage by stage in reverse:
# output norm + gate, attention, RoPE, query scale, Q/K norm + gain.  A
# gradient has its primal's dtype: with rnd=True every gradient of a bf16
# tensor is rounded to bf16 where autograd would hold it (dO, dq_hat, dk_hat,
# dv, the gradient after the rotation and after the query scale, dq, dk,
# dgate); gain gradients stay in full precision; the softmax correction
# delta is formed from the stored bf16 attention output, as the fused
# SDPA/TE backward kernels do.  rnd=False gives the exact derivative of the
# unrounded forward (pinned against torch autograd).
# --------------------------------------------------------------------------

def _maybe_bf16(x, rnd):
    return round_bf16(x) if rnd else np.asarray(x, dtype=np.float64)


def out_norm_gate_bwd(o, gate, dout, eps, rnd=True):
    """Gradients of out = normalize(o) * sigmoid(gate): returns (do, dgate).

    With y = o r, r = (mean(o^2) + eps)^-1/2, s = sigmoid(gate):
    dgate = dout y s (1 - s); dy = dout s; do = r dy - r^3 o mean(dy o).
    """
    o = np.asarray(o, dtype=np.float64)
    g = np.asarray(gate, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    y, r = rms_normalize(o, eps)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-g))
    dgate = dout * y * s * (1.0 - s)
    dy = dout * s
    r = r[..., None]
    do = r * dy - r ** 3 * o * np.mean(dy * o, axis=-1, keepdims=True)
    return _maybe_bf16(do, rnd), _maybe_bf16(dgate, rnd)


def attention_bwd(q_hat, k_hat, v, d_o, segments: Segments, *, window=0, scaling, causal=True,
                  key_valid=None, rnd=True, o=None, mags=False, d_o_abs=None):
    """Gradients of o = softmax(scaling q k^T, masked) v per segment and head.

    With P the softmax, dP = dO v^T, delta_i = sum_j P_ij dP_ij and
    dS = P (dP - delta): dq = scaling dS k, dk = scaling dS^T q, dv = P^T dO;
    a key/value head sums the contributions of its query heads.  Returns
    (dq_hat [N,Hq,D], dk_hat [N,Hkv,D], dv [N,Hkv,D]).

    ``o`` given: delta_i = sum_d dO_id o_id from that attention output, as the
    fused SDPA / Transformer Engine backward kernels the pages run form it
    from the stored (bf16) output; sum_j P_ij dP_ij equals it for the exact o.

    mags=True also returns the same sums taken over magnitudes (the scale of
    the rounding error of each result, for tolerances): with
    |dS| <= P (|dO| |v|^T + |delta|), dq_abs = scaling |dS| |k|,
    dk_abs = scaling |dS|^T |q|, dv_abs = P^T |dO|; ``d_o_abs`` replaces |dO|
    by a magnitude bound of an upstream result.
    """
    q_hat = np.asarray(q_hat, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_o = np.asarray(d_o, dtype=np.float64)
    n, hq, d = q_hat.shape
    hkv = k_hat.shape[1]
    groups = hq // hkv
    dq = np.zeros_like(q_hat)
    dk = np.zeros_like(k_hat)
    dv = np.zeros_like(v)
    if mags:
        dqa, dka, dva = np.zeros_like(q_hat), np.zeros_like(k_hat), np.zeros_like(v)
        doa_all = np.abs(d_o) if d_o_abs is None else np.asarray(d_o_abs, dtype=np.float64)
    for s0, length in zip(segments.starts, segments.lengths):
        if length == 0:
            continue
        kok = None if key_valid is None else np.asarray(key_valid)[s0:s0 + length]
        vis = visible_mask(np.arange(length), np.arange(length), window, causal, kok)
        seen = vis.any(axis=1)
        for h in range(hq):
            g = h // groups
            qs, ks, vs = q_hat[s0:s0 + length, h], k_hat[s0:s0 + length, g], v[s0:s0 + length, g]
            dos = d_o[s0:s0 + length, h]
            sc = np.where(vis, float(scaling) * (qs @ ks.T), -np.inf)
            mx = np.where(seen, sc.max(axis=1, initial=-np.inf), 0.0)[:, None]
            e = np.where(vis, np.exp(sc - mx), 0.0)
            z = e.sum(axis=1, keepdims=True)
            p = e / np.where(z > 0, z, 1.0)
            dp = dos @ vs.T
            if o is None:
                delta = np.sum(p * dp, axis=1, keepdims=True)
            else:
                delta = np.sum(dos * np.asarray(o, dtype=np.float64)[s0:s0 + length, h], axis=1,
                               keepdims=True)
            ds = p * (dp - delta)
            dq[s0:s0 + length, h] = float(scaling) * (ds @ ks)
            dk[s0:s0 + length, g] += float(scaling) * (ds.T @ qs)
            dv[s0:s0 + length, g] += p.T @ dos
            if mags:
                doa = doa_all[s0:s0 + length, h]
                oa = np.abs(dp) if o is None else np.abs(np.asarray(o, dtype=np.float64)[s0:s0 + length, h])
                da = (doa @ np.abs(vs).T)
                dla = (np.sum(p * da, axis=1, keepdims=True) if o is None
                       else np.sum(doa * oa, axis=1, keepdims=True))
                dsa = p * (da + dla)
                dqa[s0:s0 + length, h] = float(scaling) * (dsa @ np.abs(ks))
                dka[s0:s0 + length, g] += float(scaling) * (dsa.T @ np.abs(qs))
                dva[s0:s0 + length, g] += p.T @ doa
    out = (_maybe_bf16(dq, rnd), _maybe_bf16(dk, rnd), _maybe_bf16(dv, rnd))
    return out + (dqa, dka, dva) if mags else out


def rope_rotate_bwd(dy, cos, sin, upcast: bool = True):
    """Transpose of the rotation: each pair's gradient rotated back,
    (dy0 C + dy1 S, -dy0 S + dy1 C), unrounded.

    upcast=False (the Q/K-dtype rotation): C and S are the bf16 casts the
    forward rotates with, and the bf16 roundings of its products and sums are
    taken as the identity (their derivative almost everywhere), so the
    gradient is the transpose of the rotation by bf16(C), bf16(S).
    """
    if not upcast:
        cos = round_bf16(np.asarray(cos, dtype=np.float64))
        sin = round_bf16(np.asarray(sin, dtype=np.float64))
    dy = np.asarray(dy, dtype=np.float64)
    d0, d1 = dy[..., 0::2], dy[..., 1::2]
    dx = np.empty_like(dy)
    dx[..., 0::2] = d0 * cos + d1 * sin
    dx[..., 1::2] = -d0 * sin + d1 * cos
    return dx


def rms_norm_bwd(x, dy, eps, gain=None, gain_center=1.0):
    """Gradients of y = x r w (r = (mean(x^2) + eps)^-1/2, w = f32(gain_center + g)):
    returns (dx unrounded, dgain summed over every row, or None without a gain).

    dgain = sum over rows of dy x r; with u = dy w: dx = r u - r^3 x mean(u x).
    """
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    xn, r = rms_normalize(x, eps)
    r = r[..., None]
    if gain is not None:
        w = round_f32(np.float64(round_f32(gain_center)) + np.asarray(gain, dtype=np.float64))
        dgain = np.sum((dy * xn).reshape(-1, x.shape[-1]), axis=0)
        u = dy * w
    else:
        dgain = None
        u = dy
    dx = r * u - r ** 3 * x * np.mean(u * x, axis=-1, keepdims=True)
    return dx, dgain


def qk_norm_rope_bwd(q, k, dq_hat, dk_hat, *, eps, q_gain=None, k_gain=None, gain_center=1.0,
                     query_scale=1.0, use_rope=True, cos=None, sin=None, normalize=True, rnd=True,
                     upcast_rope=True):
    """Gradients through _qk_norm_rope_core: returns (dq, dk, dq_gain, dk_gain).
    ``cos``/``sin`` are the per-token rows [N, D/2]; upcast_rope as rope_rotate_bwd's
    upcast."""
    dq1 = np.asarray(dq_hat, dtype=np.float64)
    dk1 = np.asarray(dk_hat, dtype=np.float64)
    if use_rope:
        c = np.asarray(cos, dtype=np.float64)[:, None, :]
        s = np.asarray(sin, dtype=np.float64)[:, None, :]
        dq1 = _maybe_bf16(rope_rotate_bwd(dq1, c, s, upcast_rope), rnd)
        dk1 = _maybe_bf16(rope_rotate_bwd(dk1, c, s, upcast_rope), rnd)
    dq1 = _maybe_bf16(dq1 * np.float64(round_f32(query_scale)), rnd)
    if not normalize:
        return dq1, dk1, None, None
    dq, dqg = rms_norm_bwd(q, dq1, eps, q_gain, gain_center)
    dk, dkg = rms_norm_bwd(k, dk1, eps, k_gain, gain_center)
    return _maybe_bf16(dq, rnd), _maybe_bf16(dk, rnd), dqg, dkg


def attn_core_bwd(q, k, v, gate, dout, segments: Segments, *, theta, eps, out_eps, scaling,
                  window=0, use_rope=True, q_gain=None, k_gain=None, gain_center=1.0,
                  query_scale=1.0, position_ids=None, causal=True, key_valid=None, rnd=True,
                  upcast_rope=True):
    """The whole backward: recomputes the forward (with the rotation upcast_rope
    selects; the Q/K-dtype one differentiated as rope_rotate_bwd states), then returns a dict
    with dq, dk, dv, dgate (bf16 values when rnd), dq_gain, dk_gain, and the forward's
    o and lse, plus the intermediate d_o, dq_hat and dk_hat.

    With rnd=False the forward is evaluated without any rounding, so the result
    is the exact derivative of the real-valued composition.
    """
    d = q.shape[-1]
    pos = segments.local_positions() if position_ids is None else np.asarray(position_ids)
    cos, sin = rope_cos_sin(theta, d, pos) if use_rope else (None, None)
    if rnd:
        fw = attn_core(q, k, v, gate, segments, theta=theta, eps=eps, out_eps=out_eps,
                       scaling=scaling, window=window, use_rope=use_rope, q_gain=q_gain,
                       k_gain=k_gain, gain_center=gain_center, query_scale=query_scale,
                       position_ids=position_ids, causal=causal, key_valid=key_valid,
                       upcast_rope=upcast_rope)
        q_hat, k_hat, o, lse = fw["q_hat"], fw["k_hat"], fw["o"], fw["lse"]
    else:
        q_hat, k_hat, o, lse = _exact_forward(q, k, v, segments, eps=eps, scaling=scaling,
                                              window=window, use_rope=use_rope, cos=cos, sin=sin,
                                              q_gain=q_gain, k_gain=k_gain, gain_center=gain_center,
                                              query_scale=query_scale, causal=causal,
                                              key_valid=key_valid, upcast_rope=upcast_rope)
    d_o, dgate = out_norm_gate_bwd(o, gate, dout, out_eps, rnd)
    dq_hat, dk_hat, dv = attention_bwd(q_hat, k_hat, v, d_o, segments, window=window, scaling=scaling,
                                       causal=causal, key_valid=key_valid, rnd=rnd, o=o if rnd else None)
    dq, dk, dqg, dkg = qk_norm_rope_bwd(q, k, dq_hat, dk_hat, eps=eps, q_gain=q_gain, k_gain=k_gain,
                                        gain_center=gain_center, query_scale=query_scale,
                                        use_rope=use_rope, cos=cos, sin=sin, rnd=rnd,
                                        upcast_rope=upcast_rope)
    return dict(dq=dq, dk=dk, dv=dv, dgate=dgate, dq_gain=dqg, dk_gain=dkg, o=o, lse=lse,
                d_o=d_o, dq_hat=dq_hat, dk_hat=dk_hat)


def _exact_forward(q, k, v, segments, *, eps, scaling, window, use_rope, cos, sin, q_gain, k_gain,
                   gain_center, query_scale, causal, key_valid, upcast_rope=True):
    """The forward with no rounding anywhere (for the exact-derivative mode); the
    Q/K-dtype rotation keeps only its bf16 cos/sin (the rotation it applies)."""
    def norm(x, gain):
        y, _ = rms_normalize(x, eps)
        if gain is not None:
            y = y * round_f32(np.float64(round_f32(gain_center)) + np.asarray(gain, dtype=np.float64))
        return y

    def rot(x):
        c = np.asarray(cos, dtype=np.float64)[:, None, :]
        s = np.asarray(sin, dtype=np.float64)[:, None, :]
        if not upcast_rope:
            c, s = round_bf16(c), round_bf16(s)
        y = np.empty_like(x)
        y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
        y[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
        return y

    q1 = norm(q, q_gain) * np.float64(round_f32(query_scale))
    k1 = norm(k, k_gain)
    if use_rope:
        q1, k1 = rot(q1), rot(k1)
    n, hq, d = q1.shape
    groups = hq // k1.shape[1]
    o = np.zeros_like(q1)
    lse = np.zeros((n, hq))
    for s0, length in zip(segments.starts, segments.lengths):
        if length == 0:
            continue
        kok = None if key_valid is None else np.asarray(key_valid)[s0:s0 + length]
        for h in range(hq):
            ob, lb = _attend_block(q1[s0:s0 + length, h], k1[s0:s0 + length, h // groups],
                                   np.asarray(v, dtype=np.float64)[s0:s0 + length, h // groups],
                                   np.arange(length), window, scaling, causal, kok)
            o[s0:s0 + length, h] = ob
            lse[s0:s0 + length, h] = lb
    return q1, k1, o, lse


def attention_bwd_rows(q_hat_rows, k_hat, v, d_o_rows, o_rows, segments: Segments, rows, *, num_heads,
                       window=0, scaling, causal=True, key_valid=None):
    """dq_hat of selected (token, head) rows, each from its own row of the
    softmax: dq = scaling sum_j P_j (dP_j - delta) k_j with delta = dO . o
    (o the stored output of that row).  Returns bf16 values [len(rows), D]."""
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    groups = num_heads // k_hat.shape[1]
    dq = np.zeros((len(rows), k_hat.shape[2]))
    for r, (t, h) in enumerate(rows):
        s0, length = segments.locate(int(t))
        g = int(h) // groups
        ks, vs = k_hat[s0:s0 + length, g], v[s0:s0 + length, g]
        kok = None if key_valid is None else np.asarray(key_valid)[s0:s0 + length]
        vis = visible_mask(np.array([int(t) - s0]), np.arange(length), window, causal, kok)[0]
        if not vis.any():
            continue
        sc = np.where(vis, float(scaling) * (ks @ np.asarray(q_hat_rows[r], dtype=np.float64)), -np.inf)
        p = np.exp(sc - sc.max())
        p /= p.sum()
        dor = np.asarray(d_o_rows[r], dtype=np.float64)
        dp = vs @ dor
        delta = float(dor @ np.asarray(o_rows[r], dtype=np.float64))
        dq[r] = float(scaling) * ((p * (dp - delta)) @ ks)
    return round_bf16(dq)


def attention_bwd_keys(q_hat, k_hat, v, d_o, o, segments: Segments, keys, *, window=0, scaling, causal=True,
                       key_valid=None, row_block=1024):
    """dk_hat and dv of selected (token, kv head) keys: the column of every
    softmax row (of the group's query heads) that sees the key, each row
    normalised over all its own keys; delta from the stored output o.
    Returns bf16 values ([len(keys), D], [len(keys), D])."""
    q_hat = np.asarray(q_hat, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_o = np.asarray(d_o, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    hq, hkv = q_hat.shape[1], k_hat.shape[1]
    groups = hq // hkv
    dk = np.zeros((len(keys), k_hat.shape[2]))
    dv = np.zeros((len(keys), k_hat.shape[2]))
    for r, (t, g) in enumerate(keys):
        s0, length = segments.locate(int(t))
        j = int(t) - s0
        kok = None if key_valid is None else np.asarray(key_valid)[s0:s0 + length]
        if kok is not None and not kok[j]:
            continue
        ks, vs = k_hat[s0:s0 + length, g], v[s0:s0 + length, g]
        # the rows that can see key j
        if causal:
            lo_i, hi_i = j, (length if not window or window <= 0 else min(length, j + window))
        else:
            lo_i, hi_i = 0, length
        for h in range(g * groups, (g + 1) * groups):
            for r0 in range(lo_i, hi_i, row_block):
                r1 = min(hi_i, r0 + row_block)
                qb = q_hat[s0 + r0:s0 + r1, h]
                vis = visible_mask(np.arange(r0, r1), np.arange(length), window, causal, kok)
                sc = np.where(vis, float(scaling) * (qb @ ks.T), -np.inf)
                seen = vis.any(axis=1)
                mx = np.where(seen, sc.max(axis=1, initial=-np.inf), 0.0)[:, None]
                e = np.where(vis, np.exp(sc - mx), 0.0)
                z = e.sum(axis=1)
                pj = np.where(seen, e[:, j] / np.where(z > 0, z, 1.0), 0.0)
                dob = d_o[s0 + r0:s0 + r1, h]
                dpj = dob @ vs[j]
                delta = np.sum(dob * o[s0 + r0:s0 + r1, h], axis=1)
                dsj = pj * (dpj - delta)
                dk[r] += float(scaling) * (dsj @ qb)
                dv[r] += pj @ dob
    return round_bf16(dk), round_bf16(dv)
