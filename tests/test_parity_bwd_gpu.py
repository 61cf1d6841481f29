"""GPU parity of the backward entry points against the FP64 oracle's backward.

Stage tests feed the oracle the GPU's own bf16 stage inputs (as the forward
stage tests do); the whole-core test runs both sides from the raw inputs.
Bars: bf16 gradients within the row max relative error of 2e-2 (the bf16
bar of the forward); FP32 sums (delta, gain gradients) within 1e-5 of the sum
of the magnitudes of their terms -- the scale of FP32 accumulation error --
when fed the same inputs, plus for the gain gradients two bf16 ulps of their
largest term (a rounded per-row gradient may legitimately sit one ulp away
when its exact value is within FP32 error of a rounding midpoint), and within
2e-2 of their largest entry when each side starts from the raw inputs.
"""

import numpy as np
import pytest
import torch

import decoder_attention_qk_amd as m
import oracle as O
import workloads as W
from gpu_util import BF16_TOL, EPS, bits_f64, core_bwd_magnitudes, check_scaled, dev_bf16, f64, make_case
from gpu_util import check_bf16 as _check_bf16

pytestmark = pytest.mark.gpu


def check_bf16(*args, **kw):
    """The row bar on gradients; the elementwise figure is recorded, not asserted."""
    return _check_bf16(*args, elem_tol=None, **kw)

BWD = [
    W.WORKLOADS["bshd_1x128_h4kv1_d64"],
    W.small_workload("bshd_b2_s200_g4", num_heads=8, num_kv_heads=2, head_dim=128, batch=2, seqlen=200),
    W.small_workload("bshd_s300_g5_w37", num_heads=5, num_kv_heads=1, head_dim=128, seqlen=300, window=37),
    W.small_workload("bshd_s130_g1_d64", num_heads=2, num_kv_heads=2, head_dim=64, seqlen=130),
    W.small_workload("thd_g3_mixed", num_heads=6, num_kv_heads=2, head_dim=128,
                     segment_lengths=(1, 77, 0, 300, 64, 65)),
    W.small_workload("bshd_norope_d64", num_heads=4, num_kv_heads=4, head_dim=64, seqlen=160,
                     use_rope=False),
    W.small_workload("bshd_g12_w1", num_heads=12, num_kv_heads=1, head_dim=128, seqlen=90, window=1),
]
IDS = [w.name for w in BWD]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.library()


def _grad(case, tensor, std=1.0):
    return W.draw_bf16(tuple(case.q.shape), std, seed=7, workload=case.w.name, layer=0, tensor=tensor)


def _check_sum(got, ref, scale, what, tol=1e-5, flip=0.0):
    err = np.abs(got - ref)
    bound = tol * np.maximum(scale, 1e-30) + flip
    assert np.all(err <= bound), f"{what}: worst {float((err / bound).max()):.3g} of the bound"


@pytest.mark.parametrize("w", BWD[:4], ids=IDS[:4])
def test_out_norm_gate_bwd_stage(w):
    case = make_case(w)
    o = dev_bf16(W.draw_bf16(tuple(case.q.shape), 0.3, seed=1, workload=w.name, layer=0, tensor="o"))
    dout = dev_bf16(_grad(case, "dout"))
    d_o, dgate, delta = m.muse_out_norm_gate_bwd(case.params, case.layout, o, case.gate, dout)
    delta2 = m.muse_attn_bwd_delta(case.params, case.layout, o, d_o)
    torch.cuda.synchronize()
    rdo, rdg = O.out_norm_gate_bwd(f64(o), bits_f64(case.x["gate"]), f64(dout), EPS)
    s1 = check_bf16(f64(d_o), rdo, what="d_o")
    s2 = check_bf16(f64(dgate), rdg, what="dgate")
    assert s1["exact"] > 0.99 and s2["exact"] > 0.99, (s1, s2)
    terms = f64(d_o) * f64(o)
    _check_sum(f64(delta), terms.sum(-1), np.abs(terms).sum(-1), "delta")
    assert torch.equal(delta, delta2)


@pytest.mark.parametrize("w", BWD, ids=IDS)
def test_attention_bwd_stage(w):
    case = make_case(w)
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, case.layout, case.q, case.k, case.q_gain,
                                             case.k_gain, case.cos, case.sin)
    o, lse = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    d_o = dev_bf16(_grad(case, "d_o"))
    delta = m.muse_attn_bwd_delta(case.params, case.layout, o, d_o)
    dq, dk, dv = m.muse_gqa_attn_bwd(case.params, case.layout, q_hat, k_hat, case.v, d_o, lse, delta)
    torch.cuda.synchronize()
    rq, rk, rv = O.attention_bwd(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), f64(d_o), case.segs,
                                 window=case.x["window"], scaling=case.scaling, o=f64(o))
    check_bf16(f64(dq), rq, what="dq_hat")
    check_bf16(f64(dk), rk, what="dk_hat")
    check_bf16(f64(dv), rv, what="dv")


@pytest.mark.parametrize("w", BWD[:5], ids=IDS[:5])
def test_qk_norm_rope_bwd_stage(w):
    _qk_bwd_stage_check(make_case(w, query_scale=0.75 if w.name == "bshd_b2_s200_g4" else 1.0))


# the Q/K-dtype rotation (upcast_rope = 0): its backward is the transpose of
# the rotation by the bf16 cos/sin
V2 = [BWD[1], BWD[4]]


@pytest.mark.parametrize("w", V2, ids=[w.name for w in V2])
def test_qk_norm_rope_bwd_stage_qk_dtype_rotation(w):
    _qk_bwd_stage_check(make_case(w, upcast_rope=False, query_scale=0.75))


def _qk_bwd_stage_check(case):
    w = case.w
    dqh = dev_bf16(_grad(case, "dq_hat"))
    dkh = dev_bf16(W.draw_bf16(tuple(case.k.shape), 1.0, seed=7, workload=w.name, layer=0, tensor="dk_hat"))
    dq, dk, dqg, dkg = m.muse_qk_norm_rope_bwd(case.params, case.layout, case.q, case.k, case.q_gain,
                                               case.k_gain, case.cos, case.sin, dqh, dkh)
    torch.cuda.synchronize()
    kw = case.oracle_kw()
    c = s = None
    if kw["use_rope"]:
        c, s = O.rope_cos_sin(w.theta, w.head_dim, case.segs.local_positions())
    rq, rk, rqg, rkg = O.qk_norm_rope_bwd(bits_f64(case.x["q"]), bits_f64(case.x["k"]), f64(dqh), f64(dkh),
                                          eps=EPS, q_gain=kw["q_gain"], k_gain=kw["k_gain"],
                                          query_scale=kw["query_scale"], use_rope=kw["use_rope"], cos=c, sin=s,
                                          upcast_rope=kw["upcast_rope"])
    sq = check_bf16(f64(dq), rq, what="dq")
    sk = check_bf16(f64(dk), rk, what="dk")
    assert sq["exact"] > 0.99 and sk["exact"] > 0.99, (sq, sk)
    # gain gradients: FP32 sums of the same terms
    for got, ref, x, dh, gain, qs in ((dqg, rqg, case.x["q"], dqh, kw["q_gain"], kw["query_scale"]),
                                      (dkg, rkg, case.x["k"], dkh, kw["k_gain"], 1.0)):
        xs = bits_f64(x)
        xn, _ = O.rms_normalize(xs, EPS)
        g = f64(dh)
        if kw["use_rope"]:
            g = O.round_bf16(O.rope_rotate_bwd(g, c[:, None, :], s[:, None, :], kw["upcast_rope"]))
        g = O.round_bf16(g * np.float64(np.float32(qs)))
        terms = np.abs(g * xn).reshape(-1, xs.shape[-1])
        _check_sum(f64(got), ref, terms.sum(0), "gain gradient", flip=2.0 ** -7 * terms.max(0))


@pytest.mark.parametrize("w", BWD, ids=IDS)
def test_core_bwd_matches_oracle(w):
    _core_bwd_check(make_case(w))


@pytest.mark.parametrize("w", V2, ids=[w.name for w in V2])
def test_core_bwd_qk_dtype_rotation(w):
    _core_bwd_check(make_case(w, upcast_rope=False))


def _core_bwd_check(case):
    dout = dev_bf16(_grad(case, "dout"))
    res = m.muse_attn_core_bwd(case.params, case.layout, case.q, case.k, case.v, case.gate, dout,
                               case.q_gain, case.k_gain, case.cos, case.sin)
    # with the forward's o and lse given instead of recomputed: identical bits
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, case.layout, case.q, case.k, case.q_gain,
                                             case.k_gain, case.cos, case.sin)
    o, lse = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    res2 = m.muse_attn_core_bwd(case.params, case.layout, case.q, case.k, case.v, case.gate, dout,
                                case.q_gain, case.k_gain, case.cos, case.sin, o=o, lse=lse)
    torch.cuda.synchronize()
    for a, b in zip(res, res2):
        assert torch.equal(a, b)
    kw = case.oracle_kw()
    ref = O.attn_core_bwd(bits_f64(case.x["q"]), bits_f64(case.x["k"]), bits_f64(case.x["v"]),
                          bits_f64(case.x["gate"]), f64(dout), case.segs, **kw)
    dq, dk, dv, dgate, dqg, dkg = res
    mag = core_bwd_magnitudes(case, f64(dout), ref, kw)
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("dgate", dgate)):
        check_scaled(f64(got), ref[name], mag[name], name)
    # most rows are well conditioned: there the plain row bar holds as well
    for name, got in (("dv", dv), ("dgate", dgate)):
        check_bf16(f64(got), ref[name], what=name)
    for name, got in (("dq_gain", dqg), ("dk_gain", dkg)):
        check_scaled(f64(got)[None], ref[name][None], mag[name][None], name)


def test_bwd_is_deterministic():
    w = BWD[1]
    case = make_case(w)
    dout = dev_bf16(_grad(case, "dout"))
    a = m.muse_attn_core_bwd(case.params, case.layout, case.q, case.k, case.v, case.gate, dout,
                             case.q_gain, case.k_gain, case.cos, case.sin)
    b = m.muse_attn_core_bwd(case.params, case.layout, case.q, case.k, case.v, case.gate, dout,
                             case.q_gain, case.k_gain, case.cos, case.sin)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---------------------------------------------------------------- modes: bidirectional, padded keys

MODES = [
    (W.small_workload("thd_bidir_g4", num_heads=8, num_kv_heads=2, head_dim=128,
                      segment_lengths=(64, 1, 129, 200, 0, 65)), dict(bidirectional=True), None),
    (W.small_workload("bshd_bidir_d64", num_heads=4, num_kv_heads=1, head_dim=64, batch=2, seqlen=100),
     dict(bidirectional=True), None),
    (BWD[1], {}, "left"),
    (BWD[2], {}, "holes"),
    (BWD[6], {}, "holes"),
]
MODE_IDS = ["thd_bidir", "bshd_bidir_d64", "pad_left", "pad_holes_w37", "pad_holes_w1"]


def _mask(kind, batch, seqlen):
    rng = np.random.default_rng(len(kind))
    valid = np.ones((batch, seqlen), dtype=bool)
    for b in range(batch):
        if kind == "left":
            valid[b, :int(rng.integers(1, seqlen))] = False
        else:
            valid[b] = rng.random(seqlen) > 0.35
    return valid


@pytest.mark.parametrize("w,kw,pad", MODES, ids=MODE_IDS)
def test_attention_bwd_modes(w, kw, pad):
    case = make_case(w, **kw)
    valid = None
    lay = case.layout
    if pad:
        valid = _mask(pad, w.batch, w.seqlen)
        lay = m.Layout.bshd(w.batch, w.seqlen, attention_mask=torch.from_numpy(valid).cuda())
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, lay, case.q, case.k, case.q_gain, case.k_gain,
                                             case.cos, case.sin)
    o, lse = m.muse_gqa_attn_fwd(case.params, lay, q_hat, k_hat, case.v, want_lse=True)
    d_o = dev_bf16(_grad(case, "d_o"))
    delta = m.muse_attn_bwd_delta(case.params, lay, o, d_o)
    dq, dk, dv = m.muse_gqa_attn_bwd(case.params, lay, q_hat, k_hat, case.v, d_o, lse, delta)
    torch.cuda.synchronize()
    okw = dict(window=case.x["window"], scaling=case.scaling, causal=not case.params.bidirectional,
               key_valid=None if valid is None else valid.reshape(-1))
    rq, rk, rv = O.attention_bwd(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), f64(d_o), case.segs,
                                 o=f64(o), **okw)
    check_bf16(f64(dq), rq, what="dq_hat")
    check_bf16(f64(dk), rk, what="dk_hat")
    check_bf16(f64(dv), rv, what="dv")
    if valid is not None:
        # padded keys get exactly zero gradients; queries with no key get a zero dq
        flat = torch.from_numpy(~valid.reshape(-1)).cuda()
        assert torch.all(dk[flat] == 0) and torch.all(dv[flat] == 0)
        none = torch.from_numpy(~np.isfinite(f64(lse)).all(axis=1)).cuda()
        if bool(none.any()):
            assert torch.all(dq[none] == 0)
    # the whole core, end to end, on the same mode
    dout = dev_bf16(_grad(case, "dout"))
    res = m.muse_attn_core_bwd(case.params, lay, case.q, case.k, case.v, case.gate, dout, case.q_gain,
                               case.k_gain, case.cos, case.sin)
    torch.cuda.synchronize()
    ckw = case.oracle_kw()
    ckw.pop("upcast_rope")
    ref = O.attn_core_bwd(bits_f64(case.x["q"]), bits_f64(case.x["k"]), bits_f64(case.x["v"]),
                          bits_f64(case.x["gate"]), f64(dout), case.segs,
                          key_valid=None if valid is None else valid.reshape(-1), **ckw)
    mag = core_bwd_magnitudes(case, f64(dout), ref, dict(ckw, key_valid=None if valid is None else valid.reshape(-1)))
    for name, got in zip(("dq", "dk", "dv", "dgate"), res[:4]):
        check_scaled(f64(got), ref[name], mag[name], f"core {name}")
