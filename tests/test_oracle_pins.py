"""Pins of the FP64 oracle against things other than itself.

Each test ties one oracle function to a closed form, a library routine, a
hand-derived fixture under tests/golden/, or brute force on tiny inputs, so
that a plausible slip (a dropped term, a wrong sign or index, a transposed
operand, an off-by-one window) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 / f32

def _golden_bf16_cases():
    cases = []
    with open(os.path.join(GOLDEN, "bf16_rounding.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split("|")
            cases.append((eval(a), eval(b)))  # fixture is trusted, repo-owned arithmetic text
    return cases


@pytest.mark.parametrize("x,expected", _golden_bf16_cases())
def test_round_bf16_hand_cases(x, expected):
    got = float(O.round_bf16(np.array([x]))[0])
    assert got == expected or (math.isinf(expected) and got == expected)
    assert math.copysign(1.0, got) == math.copysign(1.0, expected)


def test_round_bf16_matches_torch_cast_on_fp32_inputs():
    rng = np.random.default_rng(1)
    mant = rng.standard_normal(200_000).astype(np.float32)
    expo = rng.integers(-140, 128, 200_000)
    x = np.ldexp(mant.astype(np.float64), expo).astype(np.float32)   # includes subnormals, inf
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 3.4e38, -3.4e38],
                        dtype=np.float32)
    x = np.concatenate([x, specials])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_bits_decode():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x0000, 0x8000, 0x3DCD], dtype=np.uint16)
    got = O.bf16_bits_to_f64(bits)
    exp = [1.0, -2.0, np.inf, -np.inf, 2.0 ** -133, 0.0, -0.0, 0.10009765625]
    np.testing.assert_array_equal(got, exp)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, t)


def test_round_f32_ties_to_even():
    assert O.round_f32(1.0 + 2.0 ** -24) == 1.0
    assert O.round_f32(1.0 + 2.0 ** -24 + 2.0 ** -50) == 1.0 + 2.0 ** -23
    assert O.round_f32(1.0 + 3 * 2.0 ** -24) == 1.0 + 2.0 ** -22


# ---------------------------------------------------------------- RoPE table

@pytest.mark.parametrize("theta,d", [(1.0e4, 64), (5.0e5, 128), (1.0e4, 128)])
def test_inv_freq_closed_forms(theta, d):
    inv = O.rope_inv_freq(theta, d)
    assert inv.shape == (d // 2,)
    assert inv[0] == 1.0                                   # theta**0
    # i = D/4 gives theta**(-1/2) exactly in real arithmetic
    assert inv[d // 4] == np.float32(1.0 / math.sqrt(theta))
    assert np.all(np.diff(inv) < 0)
    # exponent additivity: inv_i * inv_j = inv_{i+j} up to binary32 rounding
    for i, j in [(1, 2), (3, 5), (7, 9)]:
        assert abs(inv[i] * inv[j] / inv[i + j] - 1.0) < 3 * 2.0 ** -24


def test_inv_freq_theta_1e4_quarter_point():
    assert O.rope_inv_freq(1.0e4, 64)[16] == np.float32(0.01)


def test_rope_table_position_zero_and_pair_zero():
    pos = np.arange(0, 4096, 37)
    c, s = O.rope_cos_sin(5.0e5, 128, pos)
    assert c.shape == (len(pos), 64)
    np.testing.assert_array_equal(c[0], 1.0)
    np.testing.assert_array_equal(s[0], 0.0)
    # pair 0 has inverse frequency 1, so its angle is the position itself
    for r, p in enumerate(pos):
        assert c[r, 0] == np.float32(math.cos(p))
        assert s[r, 0] == np.float32(math.sin(p))


def test_rope_table_unit_circle_and_fp32_values():
    c, s = O.rope_cos_sin(1.0e4, 64, np.arange(0, 32768, 997))
    assert np.all(np.abs(c * c + s * s - 1.0) < 4 * 2.0 ** -24)
    np.testing.assert_array_equal(c, c.astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(s, s.astype(np.float32).astype(np.float64))


def test_rope_table_power_of_two_position_angle_is_exact_product():
    # for p = 2**k the binary32 product p*inv_i is exact: angle = p * inv_i
    inv = O.rope_inv_freq(5.0e5, 128)
    c, s = O.rope_cos_sin(5.0e5, 128, [1024])
    for i in (0, 5, 31, 63):
        a = 1024.0 * float(inv[i])
        assert c[0, i] == np.float32(math.cos(a)) and s[0, i] == np.float32(math.sin(a))


def test_rope_table_angle_is_binary32_product_like_an_fp32_module():
    # An FP32 rotary module forms angle = position(fp32) * inv_freq(fp32) in
    # binary32 arithmetic; here torch does that product, float64 does cos/sin.
    inv = torch.from_numpy(O.rope_inv_freq(5.0e5, 128).astype(np.float32))
    pos = torch.arange(0, 32768, 5, dtype=torch.float32)
    ang = (pos[:, None] * inv[None, :]).to(torch.float64)
    c, s = O.rope_cos_sin(5.0e5, 128, pos.numpy())
    np.testing.assert_array_equal(c, torch.cos(ang).to(torch.float32).double().numpy())
    np.testing.assert_array_equal(s, torch.sin(ang).to(torch.float32).double().numpy())


# ---------------------------------------------------------------- 2-D (vision) RoPE table

def test_rope_2d_table_axes_on_a_non_square_grid():
    gh, gw, d = 3, 5, 64
    c, s = O.rope_cos_sin_2d(1.0e4, d, gh, gw)
    assert c.shape == s.shape == (gh * gw, d // 2)
    q = d // 4
    for p in range(gh * gw):
        y, x = divmod(p, gw)
        # a zero coordinate leaves its half unrotated
        if y == 0:
            np.testing.assert_array_equal(c[p, :q], 1.0)
            np.testing.assert_array_equal(s[p, :q], 0.0)
        if x == 0:
            np.testing.assert_array_equal(c[p, q:], 1.0)
            np.testing.assert_array_equal(s[p, q:], 0.0)
        # pairs 0 and D/4 have inverse frequency 1: their angles are y and x
        assert c[p, 0] == np.float32(math.cos(y)) and s[p, 0] == np.float32(math.sin(y))
        assert c[p, q] == np.float32(math.cos(x)) and s[p, q] == np.float32(math.sin(x))
        # pair D/8 of each half has inverse frequency theta**(-1/2) = 0.01 in binary32
        a_y = float(np.float32(y) * np.float32(0.01))
        a_x = float(np.float32(x) * np.float32(0.01))
        assert c[p, q // 2] == np.float32(math.cos(a_y)) and s[p, q // 2] == np.float32(math.sin(a_y))
        assert c[p, q + q // 2] == np.float32(math.cos(a_x))
        assert s[p, q + q // 2] == np.float32(math.sin(a_x))
    assert np.all(np.abs(c * c + s * s - 1.0) < 4 * 2.0 ** -24)
    # the inverse frequencies decrease along each half
    c1, s1 = O.rope_cos_sin_2d(1.0e4, d, 2, 2)
    ang_y = np.arctan2(s1[2, :q], c1[2, :q])       # patch (1, 0)
    ang_x = np.arctan2(s1[1, q:], c1[1, q:])       # patch (0, 1)
    assert np.all(np.diff(ang_y) < 0) and np.allclose(ang_y, ang_x, rtol=0, atol=1e-7)


def test_rope_2d_scores_depend_on_the_2d_offset_only():
    rng = np.random.default_rng(21)
    d, gh, gw = 128, 40, 40
    qv = _bf16(rng.standard_normal(d))
    kv = _bf16(rng.standard_normal(d))
    c, s = O.rope_cos_sin_2d(1.0e4, d, gh, gw)

    def score(y1, x1, y2, x2):
        p1, p2 = y1 * gw + x1, y2 * gw + x2
        return float(O.rope_rotate(qv, c[p1], s[p1]) @ O.rope_rotate(kv, c[p2], s[p2]))

    base = score(5, 7, 2, 3)
    for y1, x1, y2, x2 in [(13, 9, 10, 5), (30, 34, 27, 30), (3, 4, 0, 0)]:
        assert abs(score(y1, x1, y2, x2) - base) < 0.05 * (abs(base) + 1.0)
    # and it depends on both offsets
    assert abs(score(6, 7, 2, 3) - base) > 1e-3
    assert abs(score(5, 8, 2, 3) - base) > 1e-3


def test_norm_free_rotation_of_the_vision_attention():
    rng = np.random.default_rng(22)
    n, hq, hkv, d = 12, 4, 2, 64
    q = _bf16(3.0 * rng.standard_normal((n, hq, d)))
    k = _bf16(rng.standard_normal((n, hkv, d)))
    # no rotation and no norm: the bf16 inputs come back unchanged (and the
    # query scale alone applies, exactly for a power of two)
    q1, k1, qr, kr = O.qk_norm_rope(q, k, eps=1e-6, use_rope=False, normalize=False)
    np.testing.assert_array_equal(q1, q)
    np.testing.assert_array_equal(k1, k)
    assert qr is None and kr is None
    q2, _, _, _ = O.qk_norm_rope(q, k, eps=1e-6, use_rope=False, normalize=False, query_scale=0.5)
    np.testing.assert_array_equal(q2, q / 2)
    # with rotation: patch (0, 0) is the identity, other patches keep each pair's norm
    c, s = O.rope_cos_sin_2d(1.0e4, d, 3, 4)
    q3, k3, _, _ = O.qk_norm_rope(q, k, eps=1e-6, cos=c, sin=s, normalize=False)
    np.testing.assert_array_equal(q3[0], q[0])
    np.testing.assert_array_equal(k3[0], k[0])
    n0 = q[..., 0::2] ** 2 + q[..., 1::2] ** 2
    n1 = q3[..., 0::2] ** 2 + q3[..., 1::2] ** 2
    assert np.all(np.abs(n1 - n0) <= 2 * 2.0 ** -7 * n0 + 1e-30)
    # and the norm really is skipped: the rows keep their RMS of about 3
    assert abs(np.sqrt(np.mean(q3 ** 2)) - 3.0) < 0.3


# ---------------------------------------------------------------- RMSNorm

def _bf16(x):
    return O.round_bf16(np.asarray(x, dtype=np.float64))


def test_rms_unit_rms_before_gain():
    x = _bf16(np.random.default_rng(2).standard_normal((50, 3, 128)) * 3.0)
    y, rstd = O.rms_normalize(x, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)
    assert rstd.shape == (50, 3)


def test_rms_eps_enters_inside_the_root():
    x = _bf16(np.random.default_rng(3).standard_normal((40, 64)) * 0.01)
    eps = 1e-4
    y, rstd = O.rms_normalize(x, eps)
    m = np.mean(x * x, axis=-1)
    epsf = float(np.float32(eps))
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(m / (m + epsf)), rtol=1e-12)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(m + epsf), rtol=1e-14)


def test_rms_constant_row_and_zero_row():
    x = np.full((2, 16), -3.0)
    x[1] = 0.0
    y, rstd = O.rms_norm(x, 1e-6)
    # constant row: output is sign(c) (gain 1), rstd = 1/sqrt(c^2 + eps)
    np.testing.assert_array_equal(y[0], -1.0)
    np.testing.assert_array_equal(y[1], 0.0)
    assert abs(rstd[0] - 1.0 / math.sqrt(9.0 + float(np.float32(1e-6)))) < 1e-15


def test_rms_axis_is_last_dim_per_head():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 4, 64))
    x[:, 1] *= 100.0
    x[:, 3] *= 0.001
    y, _ = O.rms_normalize(x, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12)


def test_rms_scale_invariance_eps0():
    x = _bf16(np.random.default_rng(5).standard_normal((16, 128)))
    a, _ = O.rms_norm(x, 0.0)
    b, _ = O.rms_norm(4.0 * x, 0.0)
    np.testing.assert_array_equal(a, b)


def test_gain_zero_centered_semantics():
    x = _bf16(np.random.default_rng(6).standard_normal((16, 64)))
    plain, _ = O.rms_norm(x, 1e-6)
    g0, _ = O.rms_norm(x, 1e-6, gain=np.zeros(64), gain_center=1.0)
    np.testing.assert_array_equal(plain, g0)                 # g = 0 keeps the effective gain 1
    g1, _ = O.rms_norm(x, 1e-6, gain=np.ones(64), gain_center=1.0)
    np.testing.assert_array_equal(g1, 2.0 * plain)           # 1 + 1 = 2: exact doubling
    # a per-dim gain scales its own column (not rows, not heads)
    g = np.linspace(-0.5, 0.5, 64)
    gd, _ = O.rms_norm(x, 1e-6, gain=g, gain_center=1.0)
    y, _ = O.rms_normalize(x, 1e-6)
    np.testing.assert_allclose(gd, y * (1.0 + g), rtol=2.0 ** -8, atol=1e-30)


# ---------------------------------------------------------------- RoPE rotation

def test_rope_rotation_is_complex_multiplication():
    rng = np.random.default_rng(7)
    x = _bf16(rng.standard_normal((32, 64)))
    ang = rng.uniform(-100, 100, (32, 32))
    c, s = np.cos(ang), np.sin(ang)
    y = O.rope_rotate(x, c, s)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * (c + 1j * s)      # RoFormer: x * e^{i m theta}
    np.testing.assert_array_equal(y[:, 0::2], _bf16(z.real))
    np.testing.assert_array_equal(y[:, 1::2], _bf16(z.imag))


def test_rope_v2_is_bf16_arithmetic_of_torch():
    # layers page, apply_rotary_embedding (upcast=False, the HF release): both
    # products rounded in the Q/K dtype before they are added.  PyTorch's own
    # bf16 tensor arithmetic (each op rounded to bf16) is the reference.
    rng = np.random.default_rng(17)
    x = _bf16(rng.standard_normal((64, 64)) * 3.0)
    ang = rng.uniform(-300, 300, (64, 32))
    c, s = np.cos(ang), np.sin(ang)
    y = O.rope_rotate(x, c, s, upcast=False)
    tb = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)
    x0, x1, tc, ts = tb(x[:, 0::2]), tb(x[:, 1::2]), tb(c), tb(s)
    np.testing.assert_array_equal(y[:, 0::2], (x0 * tc - x1 * ts).double().numpy())
    np.testing.assert_array_equal(y[:, 1::2], (x0 * ts + x1 * tc).double().numpy())


def test_rope_v2_identity_at_position_zero_and_close_to_fp32_rotation():
    rng = np.random.default_rng(18)
    x = _bf16(rng.standard_normal((64, 4, 128)))
    c, s = O.rope_cos_sin(5.0e5, 128, np.zeros(64))
    np.testing.assert_array_equal(O.rope_rotate(x, c[:, None], s[:, None], upcast=False), x)
    c, s = O.rope_cos_sin(5.0e5, 128, np.arange(64) * 97)
    y1 = O.rope_rotate(x, c[:, None], s[:, None])
    y2 = O.rope_rotate(x, c[:, None], s[:, None], upcast=False)
    # the v2 path rounds C, S, both products and the sum: a few bf16 ulps of the pair norm
    nrm = np.sqrt(x[..., 0::2] ** 2 + x[..., 1::2] ** 2)
    for j in (0, 1):
        assert np.all(np.abs(y2[..., j::2] - y1[..., j::2]) <= 4 * 2.0 ** -8 * nrm + 1e-30)
    assert np.mean(y2 != y1) > 0.05      # and it is a different rounding, not the FP32 path


def test_rope_adjacent_pair_equals_split_half_after_row_permutation():
    # adapter page, _permute_rope_rows: adjacent-pair and split-half RoPE differ
    # by a permutation of head rows.  Split-half uses rotate_half(x) = [-x2, x1].
    d = 64
    rng = np.random.default_rng(8)
    x = _bf16(rng.standard_normal((10, d)))
    ang = rng.uniform(0, 50, (10, d // 2))
    c, s = np.cos(ang), np.sin(ang)
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])  # adjacent -> split-half
    xs = x[:, perm]
    half = np.concatenate([-xs[:, d // 2:], xs[:, :d // 2]], axis=1)
    ys = _bf16(xs * np.concatenate([c, c], 1) + half * np.concatenate([s, s], 1))
    y = O.rope_rotate(x, c, s)
    np.testing.assert_array_equal(y[:, perm], ys)


def test_rope_position_zero_identity_and_norm_preservation():
    rng = np.random.default_rng(9)
    x = _bf16(rng.standard_normal((64, 4, 128)))
    c, s = O.rope_cos_sin(5.0e5, 128, np.zeros(64))
    np.testing.assert_array_equal(O.rope_rotate(x, c[:, None], s[:, None]), x)
    c, s = O.rope_cos_sin(5.0e5, 128, np.arange(64) * 251)
    y = O.rope_rotate(x, c[:, None], s[:, None])
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.all(np.abs(n1 - n0) <= 2 * 2.0 ** -7 * n0 + 1e-30)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(10)
    q = _bf16(rng.standard_normal(128))
    k = _bf16(rng.standard_normal(128))

    def score(m, n):
        cm, sm = O.rope_cos_sin(1.0e4, 128, [m])
        cn, sn = O.rope_cos_sin(1.0e4, 128, [n])
        return float(O.rope_rotate(q, cm[0], sm[0]) @ O.rope_rotate(k, cn[0], sn[0]))

    base = score(7, 3)
    for m, n in [(104, 100), (1004, 1000), (12, 8)]:
        assert abs(score(m, n) - base) < 0.05 * (abs(base) + 1.0)
    assert abs(score(9, 3) - base) > 1e-3     # and it does depend on m - n


def test_qk_norm_rope_query_scale_and_gain_routing():
    rng = np.random.default_rng(11)
    n, hq, hkv, d = 6, 4, 2, 64
    q = _bf16(rng.standard_normal((n, hq, d)))
    k = _bf16(rng.standard_normal((n, hkv, d)))
    c, s = O.rope_cos_sin(1.0e4, d, np.arange(n))
    qg = np.full(d, 1.0)       # effective Q gain 2
    kg = np.full(d, -0.5)      # effective K gain 1/2
    a = O.qk_norm_rope(q, k, eps=1e-6, cos=c, sin=s)
    b = O.qk_norm_rope(q, k, eps=1e-6, cos=c, sin=s, q_gain=qg, k_gain=kg, query_scale=2.0)
    np.testing.assert_array_equal(b[0], 4.0 * a[0])     # gain 2 then scale 2
    np.testing.assert_array_equal(b[1], 0.5 * a[1])
    nr = O.qk_norm_rope(q, k, eps=1e-6, use_rope=False)
    np.testing.assert_array_equal(nr[0], O.rms_norm(q, 1e-6)[0])
    np.testing.assert_array_equal(nr[1], O.rms_norm(k, 1e-6)[0])


# ---------------------------------------------------------------- attention

def _brute_attention(q, k, v, seg_bounds, window, scaling, causal=True, valid=None):
    """Pure-Python softmax attention: query i sees the `window` most recent keys
    up to and including itself (all earlier keys when window == 0), or, when
    not causal, every key of its segment; with `valid` (per token) padded keys
    drop out, and a query left with no key gets zeros and lse = -inf."""
    n, hq, d = q.shape
    hkv = k.shape[1]
    o = np.zeros((n, hq, d))
    lse = np.zeros((n, hq))
    for (s0, length) in seg_bounds:
        for i in range(length):
            first = 0 if window <= 0 else max(0, i - window + 1)
            keys = list(range(first, i + 1)) if causal else list(range(length))
            if valid is not None:
                keys = [j for j in keys if valid[s0 + j]]
            if not keys:
                lse[s0 + i, :] = -math.inf
                continue
            for h in range(hq):
                g = h * hkv // hq
                sc = [scaling * sum(q[s0 + i, h, t] * k[s0 + j, g, t] for t in range(d)) for j in keys]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                z = sum(w)
                for t in range(d):
                    o[s0 + i, h, t] = sum(w[a] * v[s0 + j, g, t] for a, j in enumerate(keys)) / z
                lse[s0 + i, h] = mx + math.log(z)
    return o, lse


@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 1), (4, 2), (4, 1), (5, 1), (8, 8)])
@pytest.mark.parametrize("window", [0, 1, 2, 5])
def test_attention_brute_force_bshd(hq, hkv, window):
    rng = np.random.default_rng(100 + hq * 10 + window)
    b, sl, d = 2, 9, 4
    q = _bf16(rng.standard_normal((b * sl, hq, d)))
    k = _bf16(rng.standard_normal((b * sl, hkv, d)))
    v = _bf16(rng.standard_normal((b * sl, hkv, d)))
    o, lse = O.attention(q, k, v, O.Segments.bshd(b, sl), window=window, scaling=0.7)
    ro, rl = _brute_attention(q, k, v, [(0, sl), (sl, sl)], window, 0.7)
    np.testing.assert_array_equal(o, _bf16(ro))
    np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=1e-13)


def test_attention_brute_force_thd_with_length_one_segments():
    rng = np.random.default_rng(12)
    lens = [1, 5, 1, 7, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    n, hq, hkv, d = cu[-1], 4, 2, 6
    q = _bf16(rng.standard_normal((n, hq, d)))
    k = _bf16(rng.standard_normal((n, hkv, d)))
    v = _bf16(rng.standard_normal((n, hkv, d)))
    for window in (0, 2):
        o, lse = O.attention(q, k, v, O.Segments.thd(cu), window=window, scaling=0.5)
        ro, rl = _brute_attention(q, k, v, list(zip(cu[:-1], lens)), window, 0.5)
        np.testing.assert_array_equal(o, _bf16(ro))
        np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=1e-13)


def test_bidirectional_attention_brute_force_thd():
    # vision page, MuseSparkVisionAttention: packed bidirectional attention
    rng = np.random.default_rng(21)
    lens = [1, 6, 2, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    n, hq, hkv, d = cu[-1], 4, 2, 5
    q = _bf16(rng.standard_normal((n, hq, d)))
    k = _bf16(rng.standard_normal((n, hkv, d)))
    v = _bf16(rng.standard_normal((n, hkv, d)))
    o, lse = O.attention(q, k, v, O.Segments.thd(cu), scaling=0.6, causal=False)
    ro, rl = _brute_attention(q, k, v, list(zip(cu[:-1], lens)), 0, 0.6, causal=False)
    np.testing.assert_array_equal(o, _bf16(ro))
    np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=1e-13)


def test_bidirectional_attention_invariants():
    rng = np.random.default_rng(22)
    sl, hq, d = 12, 2, 8
    q = _bf16(rng.standard_normal((sl, hq, d)))
    k = _bf16(rng.standard_normal((sl, 1, d)))
    v = _bf16(rng.standard_normal((sl, 1, d)))
    segs = O.Segments.bshd(1, sl)
    o, lse = O.attention(q, k, v, segs, scaling=0.5, causal=False)
    # permuting the tokens of a segment permutes the outputs (no order anywhere)
    perm = rng.permutation(sl)
    op, lp = O.attention(q[perm], k[perm], v[perm], segs, scaling=0.5, causal=False)
    np.testing.assert_array_equal(op, o[perm])
    np.testing.assert_allclose(lp, lse[perm], rtol=1e-13)
    # the last query of a segment sees every key in both modes
    oc, lc = O.attention(q, k, v, segs, scaling=0.5)
    np.testing.assert_array_equal(oc[-1], o[-1])
    # zero queries: uniform weights over the whole segment -> the mean of V
    oz, _ = O.attention(np.zeros_like(q), k, v, segs, scaling=0.5, causal=False)
    np.testing.assert_array_equal(oz[:, 0], np.broadcast_to(_bf16(v[:, 0].mean(axis=0)), (sl, d)))


@pytest.mark.parametrize("window", [0, 1, 3])
def test_padded_keys_brute_force_bshd(window):
    rng = np.random.default_rng(30 + window)
    b, sl, hq, hkv, d = 3, 10, 4, 2, 4
    q = _bf16(rng.standard_normal((b * sl, hq, d)))
    k = _bf16(rng.standard_normal((b * sl, hkv, d)))
    v = _bf16(rng.standard_normal((b * sl, hkv, d)))
    valid = np.ones(b * sl, dtype=bool)
    valid[:3] = False                   # row 0: left padding (its first queries see nothing)
    valid[sl + 7:2 * sl] = False        # row 1: right padding
    valid[2 * sl + 2] = valid[2 * sl + 5] = False   # row 2: holes
    o, lse = O.attention(q, k, v, O.Segments.bshd(b, sl), window=window, scaling=0.6, key_valid=valid)
    ro, rl = _brute_attention(q, k, v, [(0, sl), (sl, sl), (2 * sl, sl)], window, 0.6, valid=valid)
    np.testing.assert_array_equal(o, _bf16(ro))
    fin = np.isfinite(rl)
    np.testing.assert_array_equal(np.isfinite(lse), fin)
    np.testing.assert_allclose(lse[fin], rl[fin], rtol=1e-13, atol=1e-13)
    # the left-padded queries have no visible key: zero rows
    assert not fin[:3].any() and np.all(o[:3] == 0.0)


def test_padded_keys_invariants():
    rng = np.random.default_rng(31)
    b, sl, hq, d = 2, 16, 2, 8
    q = _bf16(rng.standard_normal((b * sl, hq, d)))
    k = _bf16(rng.standard_normal((b * sl, 1, d)))
    v = _bf16(rng.standard_normal((b * sl, 1, d)))
    segs = O.Segments.bshd(b, sl)
    # an all-valid mask is no mask
    o0, l0 = O.attention(q, k, v, segs, scaling=0.5)
    o1, l1 = O.attention(q, k, v, segs, scaling=0.5, key_valid=np.ones(b * sl, bool))
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(l1, l0)
    # the keys and values of padded tokens do not matter
    valid = rng.random(b * sl) > 0.3
    o2, l2 = O.attention(q, k, v, segs, scaling=0.5, key_valid=valid)
    k2, v2 = k.copy(), v.copy()
    k2[~valid] = 7.0
    v2[~valid] = -3.0
    o3, l3 = O.attention(q, k2, v2, segs, scaling=0.5, key_valid=valid)
    np.testing.assert_array_equal(o3, o2)
    np.testing.assert_array_equal(l3, l2)
    # left padding by p: the valid queries equal the unpadded sequence (with
    # its own positions) up to summation order
    p = 5
    valid = np.ones(sl, bool)
    valid[:p] = False
    one = O.Segments.bshd(1, sl)
    op, lp = O.attention(q[:sl], k[:sl], v[:sl], one, scaling=0.5, key_valid=valid)
    ou, lu = O.attention(q[p:sl], k[p:sl], v[p:sl], O.Segments.bshd(1, sl - p), scaling=0.5)
    np.testing.assert_allclose(lp[p:], lu, rtol=1e-13)
    assert np.all(np.abs(op[p:] - ou) <= 2.0 ** -8 * np.abs(ou))
    # a window counts positions, padded or not: W = 3 after a padded key at i-1
    # leaves the query with keys i-2 and i
    valid = np.ones(sl, bool)
    valid[9] = False
    vis = O.visible_mask(np.array([10]), np.arange(sl), 3, key_ok=valid)[0]
    assert list(np.nonzero(vis)[0]) == [8, 10]


def test_attention_golden_tiny():
    with open(os.path.join(GOLDEN, "attention_tiny.json")) as f:
        g = json.load(f)
    o, lse = O.attention(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]),
                         O.Segments.bshd(1, 2), window=g["window"], scaling=g["scaling"])
    np.testing.assert_allclose(o, g["expected_o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, g["expected_lse"], rtol=0, atol=1e-12)


def test_attention_window_one_returns_v_and_row_zero_returns_v0():
    rng = np.random.default_rng(13)
    n, hq, hkv, d = 40, 8, 2, 16
    q = _bf16(rng.standard_normal((n, hq, d)))
    k = _bf16(rng.standard_normal((n, hkv, d)))
    v = _bf16(rng.standard_normal((n, hkv, d)))
    o, lse = O.attention(q, k, v, O.Segments.bshd(1, n), window=1, scaling=0.25)
    rep = np.repeat(v, hq // hkv, axis=1)
    np.testing.assert_array_equal(o, rep)
    o2, _ = O.attention(q, k, v, O.Segments.bshd(2, n // 2), window=0, scaling=0.25)
    np.testing.assert_array_equal(o2[0], rep[0])
    np.testing.assert_array_equal(o2[n // 2], rep[n // 2])


def test_attention_zero_query_gives_prefix_and_window_means():
    rng = np.random.default_rng(14)
    n, d = 30, 8
    q = np.zeros((n, 2, d))
    k = _bf16(rng.standard_normal((n, 1, d)))
    v = _bf16(rng.standard_normal((n, 1, d)))
    o, lse = O.attention(q, k, v, O.Segments.bshd(1, n), window=0, scaling=1.0)
    csum = np.cumsum(v[:, 0], axis=0)
    cnt = np.arange(1, n + 1)[:, None]
    np.testing.assert_array_equal(o[:, 0], _bf16(csum / cnt))
    np.testing.assert_allclose(lse[:, 1], np.log(np.arange(1, n + 1)), rtol=1e-14)
    w = 4
    ow, lw = O.attention(q, k, v, O.Segments.bshd(1, n), window=w, scaling=1.0)
    for i in range(n):
        lo = max(0, i - w + 1)
        np.testing.assert_array_equal(ow[i, 0], _bf16(v[lo:i + 1, 0].mean(axis=0)))
        assert abs(lw[i, 0] - math.log(i + 1 - lo)) < 1e-14


def test_attention_invariants_window_ge_len_gqa_thd_lse():
    rng = np.random.default_rng(15)
    lens = [13, 4, 21]
    cu = np.concatenate([[0], np.cumsum(lens)])
    n, hq, hkv, d = cu[-1], 8, 2, 16
    q = _bf16(rng.standard_normal((n, hq, d)))
    k = _bf16(rng.standard_normal((n, hkv, d)))
    v = _bf16(rng.standard_normal((n, hkv, d)))
    seg = O.Segments.thd(cu)
    full, lfull = O.attention(q, k, v, seg, window=0, scaling=0.3)
    big, _ = O.attention(q, k, v, seg, window=max(lens), scaling=0.3)
    np.testing.assert_array_equal(full, big)                   # W >= L is full causal
    rep_k = np.repeat(k, hq // hkv, axis=1)                     # _repeat_kv to query heads
    rep_v = np.repeat(v, hq // hkv, axis=1)
    mha, _ = O.attention(q, rep_k, rep_v, seg, window=0, scaling=0.3)
    np.testing.assert_array_equal(full, mha)                   # GQA == MHA on repeated KV
    for s0, length in zip(cu[:-1], lens):                      # THD == per-segment BSHD
        part, lpart = O.attention(q[s0:s0 + length], k[s0:s0 + length], v[s0:s0 + length],
                                  O.Segments.bshd(1, length), window=0, scaling=0.3)
        np.testing.assert_array_equal(full[s0:s0 + length], part)
        np.testing.assert_array_equal(lfull[s0:s0 + length], lpart)
    # lse = log-sum-exp of the visible scores (library routine)
    t, h = cu[2] + 9, 5
    s = 0.3 * (k[cu[2]:t + 1, h // 4] @ q[t, h])
    assert abs(lfull[t, h] - scipy.special.logsumexp(s)) < 1e-12
    # head permutation inside a group permutes outputs
    perm = np.array([1, 0, 3, 2, 5, 4, 7, 6])
    pm, _ = O.attention(q[:, perm], k, v, seg, window=0, scaling=0.3)
    np.testing.assert_array_equal(pm, full[:, perm])


def test_visible_mask_window_counts_keys_including_self():
    vis = O.visible_mask(np.arange(10), np.arange(10), 3)
    np.testing.assert_array_equal(vis.sum(axis=1), [1, 2, 3, 3, 3, 3, 3, 3, 3, 3])
    assert vis[5, 5] and vis[5, 3] and not vis[5, 2] and not vis[5, 6]


# ---------------------------------------------------------------- output norm + gate

def test_out_gate_half_and_symmetry():
    rng = np.random.default_rng(16)
    o = _bf16(rng.standard_normal((20, 4, 64)))
    half, _ = O.out_norm_gate(o, np.zeros_like(o), 1e-6)
    one, _ = O.out_norm_gate(o, np.full_like(o, 40.0), 1e-6)
    np.testing.assert_array_equal(half, 0.5 * one)
    g = rng.standard_normal(o.shape) * 4.0
    a, _ = O.out_norm_gate(o, g, 0.0)
    b, _ = O.out_norm_gate(o, -g, 0.0)
    y, _ = O.rms_normalize(o, 0.0)
    np.testing.assert_allclose(a + b, y, rtol=0, atol=2 * 2.0 ** -8 * np.abs(y).max())


def test_out_gate_sigmoid_matches_library_on_unit_rows():
    g = _bf16(np.linspace(-30, 30, 128))
    o = np.full((1, 128), 2.0)               # normalises to exactly 1
    out, rstd = O.out_norm_gate(o, g[None, :], 0.0)
    np.testing.assert_array_equal(out[0], _bf16(scipy.special.expit(g)))
    assert rstd[0] == 0.5


def test_out_norm_unit_rms():
    rng = np.random.default_rng(17)
    o = _bf16(rng.standard_normal((30, 64)) * 0.05)
    out, _ = O.out_norm_gate(o, np.full_like(o, 40.0), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(out * out, axis=-1)), 1.0, rtol=2.0 ** -8)


# ---------------------------------------------------------------- composition

def test_segments_positions_restart_per_segment():
    seg = O.Segments.thd([0, 3, 3 + 5, 3 + 5 + 2])
    np.testing.assert_array_equal(seg.local_positions(), [0, 1, 2, 0, 1, 2, 3, 4, 0, 1])
    np.testing.assert_array_equal(O.Segments.bshd(2, 3).local_positions(), [0, 1, 2, 0, 1, 2])


def test_core_rows_match_full_core():
    rng = np.random.default_rng(18)
    lens = [17, 40, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    n, hq, hkv, d = cu[-1], 6, 2, 32
    q = _bf16(rng.standard_normal((n, hq, d)))
    k = _bf16(rng.standard_normal((n, hkv, d)))
    v = _bf16(rng.standard_normal((n, hkv, d)))
    gate = _bf16(rng.standard_normal((n, hq, d)))
    qg = _bf16(rng.standard_normal(d) * 0.05)
    kg = _bf16(rng.standard_normal(d) * 0.05)
    kw = dict(theta=1.0e4, eps=1e-6, out_eps=1e-6, scaling=d ** -0.5, window=7, q_gain=qg,
              k_gain=kg)
    seg = O.Segments.thd(cu)
    full = O.attn_core(q, k, v, gate, seg, **kw)
    rows = [(0, 0), (16, 5), (17, 2), (56, 3), (cu[2] + 8, 1), (30, 4)]
    tok = [t for t, _ in rows]
    hd = [h for _, h in rows]
    part = O.attn_core_rows(q[tok, hd], k, v, gate[tok, hd], seg, rows, num_heads=hq, **kw)
    for r, (t, h) in enumerate(rows):
        np.testing.assert_array_equal(part["out"][r], full["out"][t, h])
        np.testing.assert_array_equal(part["q_hat"][r], full["q_hat"][t, h])
        assert part["lse"][r] == full["lse"][t, h]
    np.testing.assert_array_equal(part["k_hat"], full["k_hat"])


@pytest.mark.parametrize("causal,window,valid", [(True, 0, False), (True, 1, False), (True, 3, False),
                                                  (True, 7, True), (False, 0, False), (False, 0, True)])
def test_grouped_rows_brute_force(causal, window, valid):
    """The grouped row evaluation against pure-Python softmax on rows spread
    over segments of mixed lengths (one of length 1), heads of several KV
    groups, blocks of a few rows, with and without padded keys."""
    rng = np.random.default_rng(31 + window + 2 * causal + 5 * valid)
    lens = [13, 1, 22, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    n, hq, hkv, d = cu[-1], 6, 2, 5
    q = _bf16(rng.standard_normal((n, hq, d)))
    k = _bf16(rng.standard_normal((n, hkv, d)))
    v = _bf16(rng.standard_normal((n, hkv, d)))
    ok = rng.random(n) > 0.3 if valid else None
    ro, rl = _brute_attention(q, k, v, list(zip(cu[:-1], lens)), window, 0.55, causal=causal, valid=ok)
    rows = [(int(t), int(h)) for t in rng.permutation(n)[:30] for h in rng.choice(hq, 2, replace=False)]
    qr = np.stack([q[t, h] for t, h in rows])
    go, gl = O.attention_rows_grouped(qr, k, v, O.Segments.thd(cu), rows, num_heads=hq, window=window,
                                      scaling=0.55, causal=causal, key_valid=ok, block=3)
    for r, (t, h) in enumerate(rows):
        np.testing.assert_array_equal(go[r], _bf16(ro[t, h]))
        assert gl[r] == rl[t, h] or abs(gl[r] - rl[t, h]) <= 1e-13 * max(1.0, abs(rl[t, h]))


def test_grouped_rows_match_per_row_evaluation_at_size():
    # many rows of a longer sequence with a window: the grouped blocks span
    # several windows
    rng = np.random.default_rng(77)
    n, hq, hkv, d = 700, 8, 2, 16
    q = _bf16(rng.standard_normal((n, hq, d)))
    k = _bf16(rng.standard_normal((n, hkv, d)))
    v = _bf16(rng.standard_normal((n, hkv, d)))
    seg = O.Segments.bshd(2, 350)
    rows = [(int(t), int(rng.integers(hq))) for t in range(0, n, 3)]
    qr = np.stack([q[t, h] for t, h in rows])
    for window in (0, 40):
        a, la = O.attention_rows(qr, k, v, seg, rows, num_heads=hq, window=window, scaling=0.25)
        b, lb = O.attention_rows_grouped(qr, k, v, seg, rows, num_heads=hq, window=window, scaling=0.25)
        assert np.max(np.abs(a - b)) <= 2.0 ** -8 * np.max(np.abs(a))   # fp64 summation order only
        assert np.mean(a == b) > 0.999
        np.testing.assert_allclose(la, lb, rtol=1e-12, atol=1e-12)


def test_rope_rotations_compose():
    # R(a) R(b) = R(a + b): two rotations by the table rows of positions a and b
    # equal one rotation by the row of a + b, up to the FP32 table and the two
    # bf16 roundings
    rng = np.random.default_rng(50)
    x = _bf16(rng.standard_normal((16, 64)))
    for a, b in [(3, 5), (100, 27), (1000, 2500)]:
        ca, sa = O.rope_cos_sin(1.0e4, 64, [a])
        cb, sb = O.rope_cos_sin(1.0e4, 64, [b])
        cab, sab = O.rope_cos_sin(1.0e4, 64, [a + b])
        two = O.rope_rotate(O.rope_rotate(x, ca[0], sa[0]), cb[0], sb[0])
        one = O.rope_rotate(x, cab[0], sab[0])
        pair = np.maximum(np.abs(one[..., 0::2]), np.abs(one[..., 1::2])).repeat(2, axis=-1)
        assert np.all(np.abs(two - one) <= 3 * 2.0 ** -8 * pair + 1e-3 * (a + b) * 2.0 ** -20)
