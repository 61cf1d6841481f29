"""Pins of the oracle's backward (CPU only).

The exact-derivative mode (rnd=False) is checked against torch autograd of
an independently written float64 forward and against central finite
differences; the rounded mode against invariants that hold for any
rounding of the gradients (closed forms, conservation laws).
"""

import math

import numpy as np
import pytest
import torch

import oracle as O


def _bf16(x):
    return O.round_bf16(np.asarray(x, dtype=np.float64))


def _mask(length, window, causal, valid):
    m = torch.zeros((length, length), dtype=torch.bool)
    for i in range(length):
        for j in range(length):
            ok = True if not causal else (j <= i and (window <= 0 or j > i - window))
            if valid is not None and not valid[j]:
                ok = False
            m[i, j] = ok
    return m


def _torch_forward(q, k, v, gate, bounds, *, eps, out_eps, scaling, window, cos, sin, q_gain, k_gain,
                   gain_center, query_scale, causal, valid):
    """out = norm(attn(rope(scale(norm(q))), rope(norm(k)), v)) * sigmoid(gate), float64,
    no rounding; written from the stage definitions, sharing nothing with the oracle."""
    e32 = float(np.float32(eps))

    def norm(x, g):
        y = x * torch.rsqrt((x * x).mean(-1, keepdim=True) + e32)
        if g is not None:
            w32 = (float(np.float32(gain_center)) + g).detach().to(torch.float32).to(torch.float64)
            y = y * (g + (w32 - g.detach()))     # value f32(c + g), derivative 1
        return y

    def rot(x):
        c, s = cos[:, None, :], sin[:, None, :]
        x0, x1 = x[..., 0::2], x[..., 1::2]
        return torch.stack((x0 * c - x1 * s, x0 * s + x1 * c), dim=-1).flatten(-2)

    qh = norm(q, q_gain) * float(np.float32(query_scale))
    kh = norm(k, k_gain)
    if cos is not None:
        qh, kh = rot(qh), rot(kh)
    hq, hkv = q.shape[1], k.shape[1]
    outs = []
    for s0, length in bounds:
        if length == 0:
            continue
        m = _mask(length, window, causal, None if valid is None else valid[s0:s0 + length])
        kk = kh[s0:s0 + length].repeat_interleave(hq // hkv, dim=1)     # [L, Hq, D]
        vv = v[s0:s0 + length].repeat_interleave(hq // hkv, dim=1)
        qq = qh[s0:s0 + length]
        sc = scaling * torch.einsum("ihd,jhd->hij", qq, kk)
        sc = sc.masked_fill(~m[None], -math.inf)
        p = torch.softmax(sc, dim=-1)
        p = torch.nan_to_num(p, nan=0.0)             # rows with no visible key
        outs.append(torch.einsum("hij,jhd->ihd", p, vv))
    o = torch.cat(outs, dim=0)
    on = o * torch.rsqrt((o * o).mean(-1, keepdim=True) + float(np.float32(out_eps)))
    return on * torch.sigmoid(gate)


CASES = [
    dict(name="bshd_causal", bounds=[(0, 7), (7, 7)], hq=4, hkv=2, window=0, causal=True, valid=None,
         rope=True, gains=True, qs=1.0),
    dict(name="bshd_window_qs", bounds=[(0, 9)], hq=3, hkv=1, window=3, causal=True, valid=None,
         rope=True, gains=True, qs=0.75),
    dict(name="thd_norope", bounds=[(0, 1), (1, 5), (6, 4)], hq=2, hkv=2, window=0, causal=True,
         valid=None, rope=False, gains=False, qs=1.0),
    dict(name="bidir", bounds=[(0, 5), (5, 6)], hq=4, hkv=1, window=0, causal=False, valid=None,
         rope=True, gains=True, qs=1.0),
    dict(name="padded", bounds=[(0, 8), (8, 8)], hq=2, hkv=1, window=2, causal=True,
         valid=np.array([0, 0, 1, 1, 0, 1, 1, 1, 1, 1, 1, 0, 1, 1, 1, 1], dtype=bool), rope=True,
         gains=True, qs=1.0),
    # the Q/K-dtype rotation: the torch side casts its own copy of the table to bf16
    dict(name="qk_dtype_rope", bounds=[(0, 6), (6, 9)], hq=4, hkv=2, window=0, causal=True, valid=None,
         rope=True, gains=True, qs=0.75, upcast=False),
]


def _inputs(case, seed, d=8):
    rng = np.random.default_rng(seed)
    n = sum(length for _, length in case["bounds"])
    x = dict(q=_bf16(rng.standard_normal((n, case["hq"], d))),
             k=_bf16(rng.standard_normal((n, case["hkv"], d))),
             v=_bf16(rng.standard_normal((n, case["hkv"], d))),
             gate=_bf16(rng.standard_normal((n, case["hq"], d))),
             dout=_bf16(rng.standard_normal((n, case["hq"], d))),
             q_gain=_bf16(0.1 * rng.standard_normal(d)) if case["gains"] else None,
             k_gain=_bf16(0.1 * rng.standard_normal(d)) if case["gains"] else None)
    segs = O.Segments([s for s, _ in case["bounds"]], [n_ for _, n_ in case["bounds"]])
    pos = segs.local_positions()
    cos, sin = O.rope_cos_sin(1.0e4, d, pos) if case["rope"] else (None, None)
    return x, segs, cos, sin


def _kw(case, x):
    return dict(theta=1.0e4, eps=1e-6, out_eps=1e-6, scaling=0.35, window=case["window"],
                use_rope=case["rope"], q_gain=x["q_gain"], k_gain=x["k_gain"], query_scale=case["qs"],
                causal=case["causal"], key_valid=case["valid"], upcast_rope=case.get("upcast", True))


def _torch_table(t, case):
    """The table the rotation multiplies by: as given, or cast to bf16 by torch."""
    if t is None:
        return None
    t = torch.tensor(t)
    return t if case.get("upcast", True) else t.to(torch.float32).to(torch.bfloat16).to(torch.float64)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_exact_backward_matches_torch_autograd(case):
    x, segs, cos, sin = _inputs(case, 40)
    ref = O.attn_core_bwd(x["q"], x["k"], x["v"], x["gate"], x["dout"], segs, rnd=False, **_kw(case, x))
    t = {kk: (torch.tensor(vv, dtype=torch.float64, requires_grad=True) if vv is not None else None)
         for kk, vv in x.items() if kk != "dout"}
    out = _torch_forward(t["q"], t["k"], t["v"], t["gate"], case["bounds"], eps=1e-6, out_eps=1e-6,
                         scaling=0.35, window=case["window"],
                         cos=_torch_table(cos, case), sin=_torch_table(sin, case),
                         q_gain=t["q_gain"], k_gain=t["k_gain"], gain_center=1.0,
                         query_scale=case["qs"], causal=case["causal"], valid=case["valid"])
    (out * torch.tensor(x["dout"])).sum().backward()
    pairs = [("dq", "q"), ("dk", "k"), ("dv", "v"), ("dgate", "gate")]
    if case["gains"]:
        pairs += [("dq_gain", "q_gain"), ("dk_gain", "k_gain")]
    for ours, theirs in pairs:
        g = t[theirs].grad.numpy()
        scale = np.abs(g).max() + 1e-30
        assert np.abs(ref[ours] - g).max() <= 1e-10 * scale, (ours, np.abs(ref[ours] - g).max(), scale)


@pytest.mark.parametrize("ci", [1, 5], ids=["fp32_rope", "qk_dtype_rope"])
def test_exact_backward_matches_finite_differences(ci):
    case = CASES[ci]
    x, segs, cos, sin = _inputs(case, 41)
    kw = _kw(case, x)
    ref = O.attn_core_bwd(x["q"], x["k"], x["v"], x["gate"], x["dout"], segs, rnd=False, **kw)

    def loss(q, k, v, gate):
        qh, kh, o, _ = O.muse_oracle._exact_forward(
            q, k, v, segs, eps=1e-6, scaling=0.35, window=case["window"], use_rope=True, cos=cos,
            sin=sin, q_gain=x["q_gain"], k_gain=x["k_gain"], gain_center=1.0, query_scale=case["qs"],
            causal=True, key_valid=None, upcast_rope=case.get("upcast", True))
        y, _ = O.rms_normalize(o, 1e-6)
        return float(np.sum(y / (1.0 + np.exp(-gate)) * x["dout"]))

    rng = np.random.default_rng(5)
    base = [x["q"], x["k"], x["v"], x["gate"]]
    for idx, name in enumerate(["dq", "dk", "dv", "dgate"]):
        direction = rng.standard_normal(base[idx].shape)
        h = 1e-6
        plus = [b.copy() for b in base]
        minus = [b.copy() for b in base]
        plus[idx] = plus[idx] + h * direction
        minus[idx] = minus[idx] - h * direction
        fd = (loss(*plus) - loss(*minus)) / (2 * h)
        an = float(np.sum(ref[name] * direction))
        assert abs(fd - an) <= 1e-6 * (abs(an) + 1.0), (name, fd, an)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_backward_conservation_laws(case):
    # Shifting every key of a segment by one vector moves each score row by a
    # constant, which softmax ignores: the key gradients of a segment sum to 0.
    # Each visible softmax row sums to 1: the value gradients of a segment sum
    # to the output gradients of its rows that see at least one key.
    x, segs, _, _ = _inputs(case, 42)
    q_hat = _bf16(np.random.default_rng(1).standard_normal(x["q"].shape))
    k_hat = _bf16(np.random.default_rng(2).standard_normal(x["k"].shape))
    d_o = x["dout"]
    dq, dk, dv = O.attention_bwd(q_hat, k_hat, x["v"], d_o, segs, window=case["window"], scaling=0.35,
                                 causal=case["causal"], key_valid=case["valid"], rnd=False)
    g = case["hq"] // case["hkv"]
    for s0, length in case["bounds"]:
        if length == 0:
            continue
        sl = slice(s0, s0 + length)
        assert np.abs(dk[sl].sum(axis=0)).max() < 1e-12
        vis = O.visible_mask(np.arange(length), np.arange(length), case["window"], case["causal"],
                             None if case["valid"] is None else case["valid"][sl])
        seen = vis.any(axis=1)
        want = d_o[sl][seen].reshape(-1, case["hkv"], g, d_o.shape[-1]).sum(axis=(0, 2))
        np.testing.assert_allclose(dv[sl].sum(axis=0), want, rtol=1e-12, atol=1e-12)
    # rows that see no key get no query gradient
    if case["valid"] is not None:
        assert np.all(dq[:2] == 0.0)


def test_out_gate_bwd_closed_forms():
    rng = np.random.default_rng(43)
    o = _bf16(rng.standard_normal((5, 3, 16)))
    dout = _bf16(rng.standard_normal((5, 3, 16)))
    y, _ = O.rms_normalize(o, 1e-6)
    do, dg = O.out_norm_gate_bwd(o, np.zeros_like(o), dout, 1e-6, rnd=False)
    np.testing.assert_allclose(dg, dout * y / 4.0, rtol=1e-14)          # sigma'(0) = 1/4
    # RMS normalisation is scale invariant: the input gradient is orthogonal to o (eps = 0)
    do0, _ = O.out_norm_gate_bwd(o, np.zeros_like(o), dout, 0.0, rnd=False)
    assert np.abs(np.sum(do0 * o, axis=-1)).max() < 1e-13
    # and rounded mode returns bf16 values
    do1, dg1 = O.out_norm_gate_bwd(o, np.zeros_like(o), dout, 1e-6)
    np.testing.assert_array_equal(do1, _bf16(do1))
    np.testing.assert_array_equal(dg1, _bf16(dg1))


def test_rms_norm_bwd_closed_forms():
    rng = np.random.default_rng(44)
    x = _bf16(rng.standard_normal((6, 2, 16)))
    dy = rng.standard_normal((6, 2, 16))
    dx, dg = O.rms_norm_bwd(x, dy, 0.0)
    assert dg is None
    assert np.abs(np.sum(dx * x, axis=-1)).max() < 1e-12            # scale invariance
    # a zero gain reduces to the gain-free case, and the gain gradient is the
    # column sum of dy times the normalised input
    dx1, dg1 = O.rms_norm_bwd(x, dy, 0.0, gain=np.zeros(16))
    np.testing.assert_allclose(dx1, dx, rtol=1e-14, atol=1e-15)
    xn = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
    np.testing.assert_allclose(dg1, np.sum(dy * xn, axis=(0, 1)), rtol=1e-12, atol=1e-12)


def test_rope_bwd_is_the_inverse_rotation():
    rng = np.random.default_rng(45)
    x = rng.standard_normal((20, 3, 64))
    c, s = O.rope_cos_sin(1.0e4, 64, np.arange(20) * 37)
    c, s = c[:, None, :], s[:, None, :]
    y = np.empty_like(x)
    y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    y[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    np.testing.assert_allclose(O.rope_rotate_bwd(y, c, s), x, rtol=0, atol=1e-6)
    # position 0: the identity
    c0, s0 = O.rope_cos_sin(1.0e4, 64, np.zeros(20))
    np.testing.assert_array_equal(O.rope_rotate_bwd(x, c0[:, None], s0[:, None]), x)


@pytest.mark.parametrize("ci", [0, 5], ids=["fp32_rope", "qk_dtype_rope"])
def test_rounded_backward_sits_near_the_exact_one(ci):
    case = CASES[ci]
    x, segs, _, _ = _inputs(case, 46, d=16)
    a = O.attn_core_bwd(x["q"], x["k"], x["v"], x["gate"], x["dout"], segs, rnd=True, **_kw(case, x))
    b = O.attn_core_bwd(x["q"], x["k"], x["v"], x["gate"], x["dout"], segs, rnd=False, **_kw(case, x))
    for name in ("dq", "dk", "dv", "dgate"):
        np.testing.assert_array_equal(a[name], _bf16(a[name]))
        err = np.abs(a[name] - b[name]).max() / np.abs(b[name]).max()
        assert err < 0.05, (name, err)
    for name in ("dq_gain", "dk_gain"):
        err = np.abs(a[name] - b[name]).max() / np.abs(b[name]).max()
        assert err < 0.05, (name, err)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_delta_from_the_exact_output_is_the_softmax_correction(case):
    # sum_j P_ij dP_ij = sum_d dO_id O_id when O = P V exactly: forming delta
    # from the attention output changes nothing but its rounding
    x, segs, _, _ = _inputs(case, 47)
    q_hat = _bf16(np.random.default_rng(3).standard_normal(x["q"].shape))
    k_hat = _bf16(np.random.default_rng(4).standard_normal(x["k"].shape))
    kw = dict(window=case["window"], scaling=0.35, causal=case["causal"], key_valid=case["valid"], rnd=False)
    o_exact = np.zeros_like(q_hat)
    groups = case["hq"] // case["hkv"]
    for s0, length in case["bounds"]:
        kok = None if case["valid"] is None else case["valid"][s0:s0 + length]
        for h in range(case["hq"]):
            ob, _ = O.muse_oracle._attend_block(q_hat[s0:s0 + length, h], k_hat[s0:s0 + length, h // groups],
                                                x["v"][s0:s0 + length, h // groups], np.arange(length),
                                                case["window"], 0.35, case["causal"], kok)
            o_exact[s0:s0 + length, h] = ob
    a = O.attention_bwd(q_hat, k_hat, x["v"], x["dout"], segs, **kw)
    b = O.attention_bwd(q_hat, k_hat, x["v"], x["dout"], segs, o=o_exact, **kw)
    for u, w_ in zip(a, b):
        np.testing.assert_allclose(u, w_, rtol=1e-10, atol=1e-12)
    # with the bf16 output only delta moves, by dO . (bf16(O) - O)
    c = O.attention_bwd(q_hat, k_hat, x["v"], x["dout"], segs, o=_bf16(o_exact), **kw)
    np.testing.assert_allclose(c[2], a[2], rtol=1e-12, atol=1e-12)      # dv does not use delta
    assert np.abs(c[0] - a[0]).max() > 0.0


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_row_and_key_subsets_match_the_full_backward(case):
    x, segs, _, _ = _inputs(case, 48)
    q_hat = _bf16(np.random.default_rng(5).standard_normal(x["q"].shape))
    k_hat = _bf16(np.random.default_rng(6).standard_normal(x["k"].shape))
    o = _bf16(np.random.default_rng(7).standard_normal(x["q"].shape))
    kw = dict(window=case["window"], scaling=0.35, causal=case["causal"], key_valid=case["valid"])
    dq, dk, dv = O.attention_bwd(q_hat, k_hat, x["v"], x["dout"], segs, o=o, **kw)
    n = q_hat.shape[0]
    rows = [(t, h) for t in range(n) for h in range(case["hq"])]
    tok = np.array([t for t, _ in rows])
    hd = np.array([h for _, h in rows])
    got = O.attention_bwd_rows(q_hat[tok, hd], k_hat, x["v"], x["dout"][tok, hd], o[tok, hd], segs, rows,
                               num_heads=case["hq"], **kw)
    np.testing.assert_allclose(got, dq[tok, hd], rtol=0, atol=1e-12)
    keys = [(t, g) for t in range(n) for g in range(case["hkv"])]
    gk, gv = O.attention_bwd_keys(q_hat, k_hat, x["v"], x["dout"], o, segs, keys, row_block=3, **kw)
    kt = np.array([t for t, _ in keys])
    kg = np.array([g for _, g in keys])
    np.testing.assert_allclose(gk, dk[kt, kg], rtol=0, atol=1e-12)
    np.testing.assert_allclose(gv, dv[kt, kg], rtol=0, atol=1e-12)
