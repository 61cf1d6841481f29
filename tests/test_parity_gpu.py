"""GPU parity: the HIP path (through the C ABI) against the FP64 oracle.

Small cases compare every element and span several tiles, ragged tails,
windows, packed segments (including empty and length-1 ones) and GQA group
sizes 1..16.  Stage tests feed the oracle the GPU's own bf16 stage inputs.
"""

import numpy as np
import pytest
import torch

import decoder_attention_qk_amd as m
import oracle as O
import workloads as W
from gpu_util import (BF16_TOL, EPS, bits_f64, check_bf16, check_fp32, dev_bf16, f64, make_case)

pytestmark = pytest.mark.gpu

SMALL = [
    W.WORKLOADS["bshd_1x128_h4kv1_d64"],
    W.small_workload("bshd_b2_s200_g4", num_heads=8, num_kv_heads=2, head_dim=128, batch=2, seqlen=200),
    W.small_workload("bshd_s300_g5_w37", num_heads=5, num_kv_heads=1, head_dim=128, seqlen=300, window=37),
    W.small_workload("bshd_s130_g1_d64", num_heads=2, num_kv_heads=2, head_dim=64, seqlen=130),
    W.small_workload("bshd_s257_g8_w64", num_heads=16, num_kv_heads=2, head_dim=128, seqlen=257, window=64),
    W.small_workload("thd_g3_mixed", num_heads=6, num_kv_heads=2, head_dim=128,
                     segment_lengths=(1, 77, 0, 300, 64, 65)),
    W.small_workload("thd_g5_w100", num_heads=40, num_kv_heads=8, head_dim=128,
                     segment_lengths=(500, 3, 129), window=100, theta=5.0e5),
    W.small_workload("bshd_norope_d64", num_heads=4, num_kv_heads=4, head_dim=64, seqlen=160,
                     use_rope=False),
    W.small_workload("bshd_g16_d64", num_heads=16, num_kv_heads=1, head_dim=64, seqlen=100),
    W.small_workload("bshd_g12_w1", num_heads=12, num_kv_heads=1, head_dim=128, seqlen=90, window=1),
    W.small_workload("bshd_g2_s96_w500", num_heads=4, num_kv_heads=2, head_dim=128, seqlen=96, window=500),
]
IDS = [w.name for w in SMALL]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.library()


def _oracle_full(case):
    return O.attn_core(bits_f64(case.x["q"]), bits_f64(case.x["k"]), bits_f64(case.x["v"]),
                       bits_f64(case.x["gate"]), case.segs, **case.oracle_kw())


# ---------------------------------------------------------------- RoPE table

@pytest.mark.parametrize("theta,d,n_pos", [(1.0e4, 64, 128), (5.0e5, 128, 4096), (5.0e5, 128, 32768)])
def test_rope_table(theta, d, n_pos):
    cos, sin = m.muse_rope_cos_sin(theta, d, n_pos)
    torch.cuda.synchronize()
    rc, rs = O.rope_cos_sin(theta, d, np.arange(n_pos))
    gc, gs = f64(cos), f64(sin)
    # the same binary32 angle, cos/sin rounded once from double: equal up to
    # rare double-rounding cases (at most 1 ulp, at most a handful of entries)
    for g, r in ((gc, rc), (gs, rs)):
        diff = g != r
        assert diff.sum() <= max(2, g.size // 1_000_000)
        if diff.any():
            ulp = np.spacing(np.abs(r[diff]).astype(np.float32)).astype(np.float64)
            assert np.all(np.abs(g[diff] - r[diff]) <= ulp)


# ---------------------------------------------------------------- stage parity

@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_qk_norm_rope_stage(w):
    case = make_case(w, query_scale=0.75 if w.name == "bshd_b2_s200_g4" else 1.0)
    q_hat, k_hat, q_rstd, k_rstd = m.muse_qk_norm_rope(
        case.params, case.layout, case.q, case.k, case.q_gain, case.k_gain, case.cos, case.sin,
        want_rstd=True)
    torch.cuda.synchronize()
    kw = case.oracle_kw()
    pos = case.segs.local_positions()
    c = s = None
    if kw["use_rope"]:
        c, s = O.rope_cos_sin(w.theta, w.head_dim, pos)
    rq, rk, rqr, rkr = O.qk_norm_rope(bits_f64(case.x["q"]), bits_f64(case.x["k"]), eps=EPS,
                                      q_gain=kw["q_gain"], k_gain=kw["k_gain"],
                                      query_scale=kw["query_scale"], use_rope=kw["use_rope"],
                                      cos=c, sin=s, upcast_rope=kw["upcast_rope"])
    sq = check_bf16(f64(q_hat), rq, what="q_hat")
    sk = check_bf16(f64(k_hat), rk, what="k_hat")
    assert sq["exact"] > 0.999 and sk["exact"] > 0.999, (sq, sk)
    check_fp32(f64(q_rstd), rqr, what="q_rstd")
    check_fp32(f64(k_rstd), rkr, what="k_rstd")


@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_attention_stage(w):
    case = make_case(w)
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, case.layout, case.q, case.k, case.q_gain,
                                             case.k_gain, case.cos, case.sin)
    o, lse = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.attention(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), case.segs,
                         window=case.x["window"], scaling=case.scaling)
    check_bf16(f64(o), ro, what="o")
    check_fp32(f64(lse), rl, floor=1.0, what="lse")


@pytest.mark.parametrize("w", SMALL[:4], ids=IDS[:4])
def test_out_norm_gate_stage(w):
    case = make_case(w)
    o_bits = W.draw_bf16(tuple(case.q.shape), 0.3, seed=1, workload=w.name, layer=0, tensor="o")
    o = dev_bf16(o_bits)
    out, rstd = m.muse_out_norm_gate(case.params, case.layout, o, case.gate, want_rstd=True)
    torch.cuda.synchronize()
    rout, rr = O.out_norm_gate(bits_f64(o_bits), bits_f64(case.x["gate"]), EPS)
    st = check_bf16(f64(out), rout, what="out")
    assert st["exact"] > 0.999, st
    check_fp32(f64(rstd), rr, what="o_rstd")


# ---------------------------------------------------------------- end to end

@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_fused_core_matches_oracle_and_unfused_chain(w):
    case = make_case(w)
    out, k_hat_f, lse_f = m.muse_attn_core_fwd(case.params, case.layout, case.q, case.k, case.v,
                                               case.gate, case.q_gain, case.k_gain, case.cos,
                                               case.sin, want_lse=True)
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, case.layout, case.q, case.k, case.q_gain,
                                             case.k_gain, case.cos, case.sin)
    o, lse = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    out_u, _ = m.muse_out_norm_gate(case.params, case.layout, o, case.gate)
    torch.cuda.synchronize()
    ref = _oracle_full(case)
    check_bf16(f64(out), ref["out"], what="fused out")
    # lse is an FP32 intermediate: judged on the GPU's own bf16 q_hat/k_hat
    _, rl = O.attention(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), case.segs,
                        window=case.x["window"], scaling=case.scaling)
    check_fp32(f64(lse_f), rl, floor=1.0, what="fused lse")
    # fused == unfused chain, bit for bit
    assert torch.equal(k_hat_f.view(torch.int16), k_hat.view(torch.int16))
    assert torch.equal(out.view(torch.int16), out_u.view(torch.int16))
    assert torch.equal(lse_f, lse)


# ---------------------------------------------------------------- v2 RoPE (upcast_rope = 0)

V2 = [SMALL[1], SMALL[2], SMALL[5], SMALL[6], SMALL[8]]
V2_IDS = [w.name for w in V2]


@pytest.mark.parametrize("w", V2, ids=V2_IDS)
def test_qk_norm_rope_stage_v2_rotation(w):
    # rotation in the Q/K dtype: C, S, both products and the sum rounded to bf16
    case = make_case(w, upcast_rope=False, query_scale=0.75 if w.name == "bshd_b2_s200_g4" else 1.0)
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, case.layout, case.q, case.k, case.q_gain,
                                             case.k_gain, case.cos, case.sin)
    torch.cuda.synchronize()
    kw = case.oracle_kw()
    c, s = O.rope_cos_sin(w.theta, w.head_dim, case.segs.local_positions())
    rq, rk, _, _ = O.qk_norm_rope(bits_f64(case.x["q"]), bits_f64(case.x["k"]), eps=EPS,
                                  q_gain=kw["q_gain"], k_gain=kw["k_gain"],
                                  query_scale=kw["query_scale"], use_rope=True, cos=c, sin=s,
                                  upcast_rope=False)
    sq = check_bf16(f64(q_hat), rq, what="q_hat v2")
    sk = check_bf16(f64(k_hat), rk, what="k_hat v2")
    assert sq["exact"] > 0.999 and sk["exact"] > 0.999, (sq, sk)
    # and it is not the FP32 rotation
    rq1, _, _, _ = O.qk_norm_rope(bits_f64(case.x["q"]), bits_f64(case.x["k"]), eps=EPS,
                                  q_gain=kw["q_gain"], k_gain=kw["k_gain"],
                                  query_scale=kw["query_scale"], use_rope=True, cos=c, sin=s)
    assert np.mean(f64(q_hat) != rq1) > 0.01


@pytest.mark.parametrize("w", V2, ids=V2_IDS)
def test_fused_core_v2_rotation(w):
    case = make_case(w, upcast_rope=False, query_scale=0.75 if w.name == "thd_g3_mixed" else 1.0)
    out, k_hat_f, lse_f = m.muse_attn_core_fwd(case.params, case.layout, case.q, case.k, case.v,
                                               case.gate, case.q_gain, case.k_gain, case.cos,
                                               case.sin, want_lse=True)
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, case.layout, case.q, case.k, case.q_gain,
                                             case.k_gain, case.cos, case.sin)
    o, lse = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    out_u, _ = m.muse_out_norm_gate(case.params, case.layout, o, case.gate)
    torch.cuda.synchronize()
    ref = _oracle_full(case)
    check_bf16(f64(out), ref["out"], what="fused out v2")
    assert torch.equal(k_hat_f.view(torch.int16), k_hat.view(torch.int16))
    assert torch.equal(out.view(torch.int16), out_u.view(torch.int16))
    assert torch.equal(lse_f, lse)


# ---------------------------------------------------------------- bidirectional (packed, no causal order)

BIDIR = [SMALL[0], SMALL[1], SMALL[3], SMALL[5], SMALL[8],
         W.small_workload("thd_bidir_g4", num_heads=8, num_kv_heads=2, head_dim=128,
                          segment_lengths=(64, 1, 129, 200, 0, 65))]
BIDIR_IDS = [w.name for w in BIDIR]


@pytest.mark.parametrize("w", BIDIR, ids=BIDIR_IDS)
def test_bidirectional_attention_stage(w):
    case = make_case(w, bidirectional=True)
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, case.layout, case.q, case.k, case.q_gain,
                                             case.k_gain, case.cos, case.sin)
    o, lse = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.attention(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), case.segs,
                         scaling=case.scaling, causal=False)
    check_bf16(f64(o), ro, what="o bidirectional")
    check_fp32(f64(lse), rl, floor=1.0, what="lse bidirectional")
    # and it is not the causal result (the first row of a segment sees every key)
    rc, _ = O.attention(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), case.segs, scaling=case.scaling)
    assert np.mean(f64(o) != rc) > 0.5


@pytest.mark.parametrize("w", BIDIR, ids=BIDIR_IDS)
def test_bidirectional_fused_core(w):
    case = make_case(w, bidirectional=True)
    out, _, lse_f = m.muse_attn_core_fwd(case.params, case.layout, case.q, case.k, case.v, case.gate,
                                         case.q_gain, case.k_gain, case.cos, case.sin, want_lse=True)
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, case.layout, case.q, case.k, case.q_gain,
                                             case.k_gain, case.cos, case.sin)
    o, lse = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    out_u, _ = m.muse_out_norm_gate(case.params, case.layout, o, case.gate)
    torch.cuda.synchronize()
    check_bf16(f64(out), _oracle_full(case)["out"], what="fused out bidirectional")
    assert torch.equal(out.view(torch.int16), out_u.view(torch.int16))
    assert torch.equal(lse_f, lse)


# ---------------------------------------------------------------- vision attention (2-D RoPE, no norm)

def _table_ulp_check(g, r):
    # the same binary32 angle, cos/sin rounded once from double: equal up to
    # rare double-rounding cases (at most 1 ulp, at most a handful of entries)
    diff = g != r
    assert diff.sum() <= max(2, g.size // 1_000_000)
    if diff.any():
        ulp = np.spacing(np.abs(r[diff]).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(g[diff] - r[diff]) <= ulp)


@pytest.mark.parametrize("theta,d,gh,gw", [(1.0e4, 64, 3, 5), (1.0e4, 128, 64, 48), (5.0e5, 128, 1, 1)])
def test_rope_table_2d(theta, d, gh, gw):
    cos, sin = m.muse_rope_cos_sin_2d(theta, d, gh, gw)
    torch.cuda.synchronize()
    rc, rs = O.rope_cos_sin_2d(theta, d, gh, gw)
    _table_ulp_check(f64(cos), rc)
    _table_ulp_check(f64(sin), rs)


VISION = [
    (64, 16, ((3, 5), (8, 8), (1, 1), (8, 8), (12, 7))),
    (128, 8, ((16, 16), (2, 9), (0, 3), (5, 5), (16, 16))),
]


@pytest.mark.parametrize("d,heads,grids", VISION, ids=["d64_h16", "d128_h8"])
def test_vision_attention_path(d, heads, grids):
    """Packed grids: 2-D RoPE on un-normalised Q/K (one table per grid shape,
    shared through position_ids), then bidirectional attention per grid."""
    theta, name = 1.0e4, f"vision_d{d}"
    lens = [h * w for h, w in grids]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = int(cu[-1])
    x = {t: W.draw_bf16((n, heads, d), 1.0, seed=0, workload=name, layer=0, tensor=t) for t in "qkv"}
    shapes = sorted({g for g in grids if g[0] * g[1] > 0})
    offs, off = {}, 0
    for g in shapes:
        offs[g] = off
        off += g[0] * g[1]
    cos = torch.empty((off, d // 2), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    for g in shapes:
        o0 = offs[g]
        m.muse_rope_cos_sin_2d(theta, d, g[0], g[1], cos[o0:o0 + g[0] * g[1]], sin[o0:o0 + g[0] * g[1]])
    pos = np.concatenate([offs.get(g, 0) + np.arange(g[0] * g[1]) for g in grids]).astype(np.int32)
    lay = m.Layout.thd(torch.from_numpy(cu).cuda(), max(lens), total_tokens=n,
                       position_ids=torch.from_numpy(pos).cuda())
    p = m.AttnParams(head_dim=d, num_heads=heads, num_key_value_heads=heads, use_rope=True,
                     bidirectional=True, skip_qk_norm=True, scaling=float(np.float32(d ** -0.5)))
    q, k, v = (dev_bf16(x[t]) for t in "qkv")
    qh, kh, qr, kr = m.muse_qk_norm_rope(p, lay, q, k, None, None, cos, sin)
    o, lse = m.muse_gqa_attn_fwd(p, lay, qh, kh, v, want_lse=True)
    torch.cuda.synchronize()
    assert qr is None and kr is None
    # oracle: the per-token rows of each grid's own 2-D table
    rc = np.zeros((n, d // 2))
    rs = np.zeros((n, d // 2))
    for g, s0, ln in zip(grids, cu[:-1], lens):
        if ln:
            rc[s0:s0 + ln], rs[s0:s0 + ln] = O.rope_cos_sin_2d(theta, d, g[0], g[1])
    rq, rk, _, _ = O.qk_norm_rope(bits_f64(x["q"]), bits_f64(x["k"]), eps=EPS, cos=rc, sin=rs,
                                  normalize=False)
    sq = check_bf16(f64(qh), rq, what="vision q rotated")
    sk = check_bf16(f64(kh), rk, what="vision k rotated")
    assert sq["exact"] > 0.999 and sk["exact"] > 0.999, (sq, sk)
    segs = O.Segments.thd(cu)
    ro, rl = O.attention(f64(qh), f64(kh), bits_f64(x["v"]), segs, scaling=p.scaling, causal=False)
    check_bf16(f64(o), ro, what="vision o")
    check_fp32(f64(lse), rl, floor=1.0, what="vision lse")


# ---------------------------------------------------------------- padded keys (BSHD attention_mask)

def _pad_mask(kind, batch, seqlen, seed=0):
    rng = np.random.default_rng(seed)
    valid = np.ones((batch, seqlen), dtype=bool)
    for b in range(batch):
        if kind == "right":
            valid[b, seqlen - int(rng.integers(1, seqlen)):] = False
        elif kind == "left":                       # leading queries see no key at all
            valid[b, :int(rng.integers(1, seqlen))] = False
        elif kind == "holes":
            valid[b] = rng.random(seqlen) > 0.35
        elif kind == "tile":                       # a whole 64-key tile of padding
            valid[b, 64:128] = False
    return valid


PADDED = [
    (SMALL[1], "right"), (SMALL[1], "left"), (SMALL[2], "holes"), (SMALL[3], "left"),
    (SMALL[4], "holes"), (SMALL[8], "tile"), (SMALL[9], "holes"),
]
PADDED_IDS = [f"{w.name}-{k}" for w, k in PADDED]


def _check_lse(got, ref, what):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin) and np.all(got[~fin] == -np.inf), what
    check_fp32(got[fin], ref[fin], floor=1.0, what=what)


@pytest.mark.parametrize("w,kind", PADDED, ids=PADDED_IDS)
def test_padded_keys_attention_stage(w, kind):
    case = make_case(w)
    valid = _pad_mask(kind, w.batch, w.seqlen, seed=len(kind))
    lay = m.Layout.bshd(w.batch, w.seqlen, attention_mask=torch.from_numpy(valid).cuda())
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, lay, case.q, case.k, case.q_gain,
                                             case.k_gain, case.cos, case.sin)
    o, lse = m.muse_gqa_attn_fwd(case.params, lay, q_hat, k_hat, case.v, want_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.attention(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), case.segs,
                         window=case.x["window"], scaling=case.scaling, key_valid=valid.reshape(-1))
    check_bf16(f64(o), ro, what=f"o padded {kind}")
    _check_lse(f64(lse), rl, f"lse padded {kind}")
    if kind == "left":
        assert (~np.isfinite(rl)).any()          # the zero-row case is exercised


@pytest.mark.parametrize("w,kind", PADDED[:4], ids=PADDED_IDS[:4])
def test_padded_keys_fused_core(w, kind):
    case = make_case(w)
    valid = _pad_mask(kind, w.batch, w.seqlen, seed=len(kind))
    lay = m.Layout.bshd(w.batch, w.seqlen, attention_mask=torch.from_numpy(valid).cuda())
    out, _, lse_f = m.muse_attn_core_fwd(case.params, lay, case.q, case.k, case.v, case.gate,
                                         case.q_gain, case.k_gain, case.cos, case.sin, want_lse=True)
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, lay, case.q, case.k, case.q_gain,
                                             case.k_gain, case.cos, case.sin)
    o, lse = m.muse_gqa_attn_fwd(case.params, lay, q_hat, k_hat, case.v, want_lse=True)
    out_u, _ = m.muse_out_norm_gate(case.params, lay, o, case.gate)
    torch.cuda.synchronize()
    ref = O.attn_core(bits_f64(case.x["q"]), bits_f64(case.x["k"]), bits_f64(case.x["v"]),
                      bits_f64(case.x["gate"]), case.segs, key_valid=valid.reshape(-1),
                      **case.oracle_kw())
    check_bf16(f64(out), ref["out"], what=f"fused out padded {kind}")
    assert torch.equal(out.view(torch.int16), out_u.view(torch.int16))
    assert torch.equal(lse_f, lse)


def test_all_valid_mask_equals_no_mask():
    w = SMALL[4]
    case = make_case(w)
    lay = m.Layout.bshd(w.batch, w.seqlen,
                        attention_mask=torch.ones((w.batch, w.seqlen), dtype=torch.uint8, device="cuda"))
    a, _, la = m.muse_attn_core_fwd(case.params, case.layout, case.q, case.k, case.v, case.gate,
                                    case.q_gain, case.k_gain, case.cos, case.sin, want_lse=True)
    b, _, lb = m.muse_attn_core_fwd(case.params, lay, case.q, case.k, case.v, case.gate,
                                    case.q_gain, case.k_gain, case.cos, case.sin, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(la, lb)


# ---------------------------------------------------------------- softmax reference moves

def _spiky_attention_inputs(seed, L, hq, hkv, d, spikes):
    """q_hat aligned (or anti-aligned) with a common direction u, k_hat small noise
    except 'spike' keys c * u, so a query's scores jump by many log2 units between
    the tiles the kernel visits (diagonal first, then downwards)."""
    rng = np.random.default_rng(seed)
    u = np.ones(d)
    sign = np.where(np.arange(hq) % 2 == 0, 1.0, -1.0)
    q = 0.3 * rng.standard_normal((L, hq, d)) + sign[None, :, None] * u
    k = 0.5 * rng.standard_normal((L, hkv, d))
    for pos, c in spikes:
        k[pos] = c * u + 0.05 * rng.standard_normal((hkv, d))
    v = rng.standard_normal((L, hkv, d))
    return [torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16) for a in (q, k, v)]


@pytest.mark.parametrize("window", [0, 100])
def test_attention_reference_moves_with_score_spikes(window):
    # raw score of a spike key for an aligned query ~ 128 c; in log2 units of the
    # softmax (scaling 128^-0.5) ~ 16.3 c: jumps of 8 .. 200 log2 units between
    # visited tiles, both below the reference-move threshold (kept with a stale
    # reference) and above it (O and the sum rescaled, or the old part flushed
    # to zero), and far below every seen score for the anti-aligned heads
    L, hq, hkv, d = 320, 4, 1, 128
    spikes = [(300, 0.5), (250, 1.0), (200, 1.5), (130, 3.0), (100, 3.0), (64, 1.2), (20, 2.0), (5, 12.0)]
    qc, kc, vc = _spiky_attention_inputs(7, L, hq, hkv, d, spikes)
    params = m.AttnParams(head_dim=d, num_heads=hq, num_key_value_heads=hkv, sliding_window=window,
                          use_rope=False, scaling=float(np.float32(d ** -0.5)))
    layout = m.Layout.bshd(1, L)
    o, lse = m.muse_gqa_attn_fwd(params, layout, qc.cuda(), kc.cuda(), vc.cuda(), want_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.attention(f64(qc), f64(kc), f64(vc), O.Segments.bshd(1, L), window=window,
                         scaling=float(np.float32(d ** -0.5)))
    check_bf16(f64(o), ro, what="o")
    check_fp32(f64(lse), rl, floor=1.0, what="lse")


# ---------------------------------------------------------------- bit-exact invariants

def test_window_one_returns_v_exactly():
    w = W.small_workload("w1", num_heads=8, num_kv_heads=2, head_dim=128, batch=2, seqlen=150, window=1)
    case = make_case(w)
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, case.layout, case.q, case.k, case.q_gain,
                                             case.k_gain, case.cos, case.sin)
    o, _ = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v)
    torch.cuda.synchronize()
    rep = case.v.repeat_interleave(4, dim=1)
    assert torch.equal(o.view(torch.int16), rep.view(torch.int16))


def test_rope_position_zero_is_identity():
    w = W.small_workload("p0", num_heads=4, num_kv_heads=2, head_dim=128, segment_lengths=(5, 9, 1))
    case = make_case(w)
    a = m.muse_qk_norm_rope(case.params, case.layout, case.q, case.k, case.q_gain, case.k_gain,
                            case.cos, case.sin)
    p2 = m.AttnParams(**{**case.params.__dict__, "use_rope": False})
    b = m.muse_qk_norm_rope(p2, case.layout, case.q, case.k, case.q_gain, case.k_gain)
    torch.cuda.synchronize()
    for start in (0, 5, 14):            # first token of each segment has position 0
        assert torch.equal(a[0][start].view(torch.int16), b[0][start].view(torch.int16))
        assert torch.equal(a[1][start].view(torch.int16), b[1][start].view(torch.int16))
    assert not torch.equal(a[0][1].view(torch.int16), b[0][1].view(torch.int16))


def test_gate_zero_halves_gate_forty():
    w = SMALL[1]
    case = make_case(w)
    o = dev_bf16(W.draw_bf16(tuple(case.q.shape), 1.0, seed=2, workload=w.name, layer=0, tensor="o"))
    half, _ = m.muse_out_norm_gate(case.params, case.layout, o, torch.zeros_like(case.gate))
    one, _ = m.muse_out_norm_gate(case.params, case.layout, o, torch.full_like(case.gate, 40.0))
    torch.cuda.synchronize()
    assert torch.equal(half.float() * 2, one.float())


def test_thd_equals_per_segment_bshd():
    lens = (70, 1, 129, 64)
    w = W.small_workload("thd_eq", num_heads=8, num_kv_heads=2, head_dim=128, segment_lengths=lens,
                         window=50)
    case = make_case(w)
    out, _, lse = m.muse_attn_core_fwd(case.params, case.layout, case.q, case.k, case.v, case.gate,
                                       case.q_gain, case.k_gain, case.cos, case.sin, want_lse=True)
    s0 = 0
    for n in lens:
        sl = slice(s0, s0 + n)
        lay = m.Layout.bshd(1, n)
        o1, _, l1 = m.muse_attn_core_fwd(case.params, lay, case.q[sl].contiguous(),
                                         case.k[sl].contiguous(), case.v[sl].contiguous(),
                                         case.gate[sl].contiguous(), case.q_gain, case.k_gain,
                                         case.cos, case.sin, want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), out[sl].view(torch.int16))
        assert torch.equal(l1, lse[sl])
        s0 += n


def test_explicit_position_ids_match_oracle():
    w = W.small_workload("posids", num_heads=4, num_kv_heads=1, head_dim=128, batch=2, seqlen=70)
    case = make_case(w)
    pos = (np.arange(140) % 70 + 1000).astype(np.int32)
    pos[75] = 5
    cos, sin = m.muse_rope_cos_sin(w.theta, 128, 2048)
    lay = m.Layout.bshd(2, 70, position_ids=torch.from_numpy(pos).cuda())
    out, _, _ = m.muse_attn_core_fwd(case.params, lay, case.q, case.k, case.v, case.gate,
                                     case.q_gain, case.k_gain, cos, sin)
    torch.cuda.synchronize()
    ref = O.attn_core(bits_f64(case.x["q"]), bits_f64(case.x["k"]), bits_f64(case.x["v"]),
                      bits_f64(case.x["gate"]), case.segs, position_ids=pos, **case.oracle_kw())
    check_bf16(f64(out), ref["out"], what="out with position_ids")


# ---------------------------------------------------------------- table built by the Q/K pass

TABLE_CASES = [
    ("bshd_b2_s200_g4", dict(), None),
    ("thd_g3_mixed", dict(), None),
    ("bshd_s130_g1_d64", dict(), None),
    ("bshd_b2_s200_g4", dict(upcast_rope=False), None),
    ("bshd_b2_s200_g4", dict(query_scale=0.75), None),
    ("bshd_b2_s200_g4", dict(), "posids"),
]


@pytest.mark.parametrize("name,kw,pos_mode", TABLE_CASES,
                         ids=[f"{n}-{'-'.join(k) or 'base'}-{p or 'implicit'}" for n, k, p in TABLE_CASES])
def test_qk_norm_rope_table_equals_two_launches(name, kw, pos_mode):
    """The one-launch table mode rotates Q and K with, and writes, exactly the
    entries muse_rope_cos_sin produces (bitwise), and leaves rows of positions
    no token has untouched."""
    w = next(x for x in SMALL if x.name == name)
    case = make_case(w, **kw)
    lay, n_pos = case.layout, case.n_pos
    if pos_mode == "posids":
        pos = (np.arange(w.tokens) * 7 % 300 + 11).astype(np.int32)
        pos[3] = pos[150]       # repeated positions
        lay = m.Layout.bshd(w.batch, w.seqlen, position_ids=torch.from_numpy(pos).cuda())
        n_pos = 400
    cos, sin = m.muse_rope_cos_sin(w.theta, w.head_dim, n_pos)
    qa, ka, qra, kra = m.muse_qk_norm_rope(case.params, lay, case.q, case.k, case.q_gain, case.k_gain,
                                           cos, sin, want_rstd=True)
    sentinel = float("nan")
    cos_t = torch.full_like(cos, sentinel)
    sin_t = torch.full_like(sin, sentinel)
    qb, kb, qrb, krb, _, _ = m.muse_qk_norm_rope_table(case.params, lay, case.q, case.k, case.q_gain,
                                                       case.k_gain, theta=w.theta, n_pos=n_pos,
                                                       cos_out=cos_t, sin_out=sin_t, want_rstd=True)
    torch.cuda.synchronize()
    assert torch.equal(qa.view(torch.int16), qb.view(torch.int16))
    assert torch.equal(ka.view(torch.int16), kb.view(torch.int16))
    assert torch.equal(qra, qrb) and torch.equal(kra, krb)
    if pos_mode == "posids":
        rows = np.unique(pos)
    else:
        rows = np.arange(w.max_seqlen)
    written = np.zeros(n_pos, dtype=bool)
    written[rows] = True
    ct, st = cos_t.cpu(), sin_t.cpu()
    assert torch.equal(ct[written], cos.cpu()[written]) and torch.equal(st[written], sin.cpu()[written])
    assert torch.isnan(ct[~written]).all() and torch.isnan(st[~written]).all()
    # K only (the attention step's form), then the fused attention reads the table
    cos_k = torch.full_like(cos, sentinel)
    sin_k = torch.full_like(sin, sentinel)
    _, kc, _, _, _, _ = m.muse_qk_norm_rope_table(case.params, lay, None, case.k, None, case.k_gain,
                                                  theta=w.theta, n_pos=n_pos, cos_out=cos_k, sin_out=sin_k)
    o1, _ = m.muse_attn_fused_fwd(case.params, lay, case.q, ka, case.v, case.gate, case.q_gain, cos, sin)
    o2, _ = m.muse_attn_fused_fwd(case.params, lay, case.q, kc, case.v, case.gate, case.q_gain, cos_k, sin_k)
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), ka.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ---------------------------------------------------------------- edge cases

def test_empty_inputs_are_noops():
    p = m.AttnParams(head_dim=128, num_heads=4, num_key_value_heads=1)
    e = torch.empty((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    ek = torch.empty((0, 1, 128), dtype=torch.bfloat16, device="cuda")
    lay = m.Layout.bshd(0, 16)
    cos, sin = m.muse_rope_cos_sin(5e5, 128, 16)
    out, _, _ = m.muse_attn_core_fwd(p, lay, e, ek, ek, e, None, None, cos, sin)
    assert out.shape == (0, 4, 128)
    cu = torch.zeros(3, dtype=torch.int32, device="cuda")
    out, _, _ = m.muse_attn_core_fwd(p, m.Layout.thd(cu, 0, total_tokens=0), e, ek, ek, e, None,
                                     None, cos, sin)
    torch.cuda.synchronize()


def test_outputs_stay_inside_their_buffers_and_runs_are_deterministic():
    w = SMALL[6]
    case = make_case(w)
    n, hq, d = case.q.shape
    guard = 4096
    big = torch.full((n * hq * d + 2 * guard,), 12345, dtype=torch.int16, device="cuda")
    lse_big = torch.full((n * hq + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
    kbig = torch.full((case.k.numel() + 2 * guard,), -3, dtype=torch.int16, device="cuda")
    out = big[guard:guard + n * hq * d].view(torch.bfloat16).view(n, hq, d)
    lse = lse_big[guard:guard + n * hq].view(n, hq)
    kh = kbig[guard:guard + case.k.numel()].view(torch.bfloat16).view(case.k.shape)
    m.muse_attn_core_fwd(case.params, case.layout, case.q, case.k, case.v, case.gate, case.q_gain,
                         case.k_gain, case.cos, case.sin, out=out, lse=lse, k_hat_out=kh)
    torch.cuda.synchronize()
    assert torch.all(big[:guard] == 12345) and torch.all(big[-guard:] == 12345)
    assert torch.all(lse_big[:guard] == 7.0) and torch.all(lse_big[-guard:] == 7.0)
    assert torch.all(kbig[:guard] == -3) and torch.all(kbig[-guard:] == -3)
    out2, _, lse2 = m.muse_attn_core_fwd(case.params, case.layout, case.q, case.k, case.v, case.gate,
                                         case.q_gain, case.k_gain, case.cos, case.sin, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse, lse2)


def test_invalid_arguments_raise():
    case = make_case(SMALL[0])
    with pytest.raises(m.MuseError):
        m.muse_attn_core_fwd(case.params, case.layout, case.q, case.k, case.v, case.gate,
                             case.q_gain, case.k_gain, case.cos, case.sin, out=case.q)
    bad = m.AttnParams(**{**case.params.__dict__, "head_dim": 96})
    with pytest.raises(m.MuseError) as ei:
        m.muse_gqa_attn_fwd(bad, case.layout, case.q, case.k, case.v)
    assert ei.value.status == m.MUSE_ERR_UNSUPPORTED
