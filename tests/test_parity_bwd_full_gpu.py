"""Full-size workloads through the attention backward on the GPU (the
launch configuration the benchmark times), checked against the oracle on
sampled outputs: dq_hat on sampled (token, head) rows (each from its own
softmax row) and dk_hat, dv on sampled keys of one KV head (every query row
that sees the key, each normalised over all its own keys).  The oracle is fed
the GPU's own stage inputs: q_hat, k_hat, the stored output o; d_o is a
seeded synthetic gradient."""

import numpy as np
import pytest
import torch

import decoder_attention_qk_amd as m
import oracle as O
import workloads as W
from gpu_util import bits_f64, dev_bf16, f64, make_case, sample_rows
from gpu_util import check_bf16 as _check_bf16

pytestmark = pytest.mark.gpu


def check_bf16(*args, **kw):
    """The row bar on gradients; the elementwise figure is recorded, not asserted."""
    return _check_bf16(*args, elem_tol=None, **kw)


FULL = [
    ("bshd_1x128_h4kv1_d64", 0),
    ("bshd_2x4096_h32kv8_d128", 0),
    ("bshd_1x16384_h32kv8_d128_w4096", 0),
    ("thd_16seg_h40kv8_d128", 0),
    ("bshd_1x32768_h64kv8_d128_mix", 0),
    ("bshd_1x32768_h64kv8_d128_mix", 3),
    ("bshd_2x4096_h4kv1_d128", 0),   # one GPU's share; its forward takes the KV split
]
# a sequence past the configurations' 32k (positions and tile offsets at their
# largest); the window keeps the oracle's per-key and per-row sums short
LONG = {
    "bshd_1x131072_h8kv2_d128_w2048": W.small_workload("bshd_1x131072_h8kv2_d128_w2048", num_heads=8,
                                                       num_kv_heads=2, head_dim=128, seqlen=131072,
                                                       window=2048, theta=5.0e5),
}
FULL += [(n, 0) for n in LONG]


def _keys(segs, window, rng, n_random=4):
    """Each segment's last key, the last key of the longest segment's first
    window (or its middle), and random keys in the last eighth of the longest
    segment -- keys whose visible rows the oracle can sum in seconds."""
    keys = set()
    for s0, n in zip(segs.starts, segs.lengths):
        if n:
            keys.add(s0 + n - 1)
    s0, n = max(zip(segs.starts, segs.lengths), key=lambda u: u[1])
    keys.add(s0 + (min(window, n) - 1 if window and window > 0 else n // 2))
    for t in rng.integers(s0 + n - max(1, n // 8), s0 + n, n_random):
        keys.add(int(t))
    return sorted(keys)


@pytest.mark.parametrize("name,layer", FULL, ids=[f"{n}-L{l}" for n, l in FULL])
def test_full_size_attention_bwd_sampled(name, layer):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = LONG[name] if name in LONG else W.WORKLOADS[name]
    print(f"[full bwd] {name} layer {layer}", flush=True)
    case = make_case(w, layer)
    p, lay = case.params, case.layout
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(p, lay, case.q, case.k, case.q_gain, case.k_gain, case.cos, case.sin)
    o, lse = m.muse_gqa_attn_fwd(p, lay, q_hat, k_hat, case.v, want_lse=True)
    d_o = dev_bf16(W.draw_bf16(tuple(case.q.shape), 1.0, seed=11, workload=name, layer=layer, tensor="d_o"))
    delta = m.muse_attn_bwd_delta(p, lay, o, d_o)
    dq, dk, dv = m.muse_gqa_attn_bwd(p, lay, q_hat, k_hat, case.v, d_o, lse, delta)
    torch.cuda.synchronize()
    win = case.x["window"]
    # dq_hat rows
    rows = sample_rows(case.segs, w.num_heads, win, n_random=64, seed=layer)
    ti = torch.tensor([t for t, _ in rows], device="cuda")
    hi = torch.tensor([h for _, h in rows], device="cuda")
    k64 = f64(k_hat)
    v64 = bits_f64(case.x["v"])
    ref = O.attention_bwd_rows(f64(q_hat[ti, hi]), k64, v64, f64(d_o[ti, hi]), f64(o[ti, hi]), case.segs, rows,
                               num_heads=w.num_heads, window=win, scaling=case.scaling)
    sq = check_bf16(f64(dq[ti, hi]), ref, what=f"{name} L{layer} dq_hat rows")
    # dk_hat, dv of sampled keys of one kv head (its query heads only, to bound memory)
    g = w.num_kv_heads - 1
    grp = w.num_heads // w.num_kv_heads
    hs = slice(g * grp, (g + 1) * grp)
    keys = _keys(case.segs, win, np.random.default_rng(layer))
    kk, kv = O.attention_bwd_keys(f64(q_hat[:, hs]), k64[:, g:g + 1], v64[:, g:g + 1], f64(d_o[:, hs]),
                                  f64(o[:, hs]), case.segs, [(t, 0) for t in keys], window=win,
                                  scaling=case.scaling)
    kt = torch.tensor(keys, device="cuda")
    sk = check_bf16(f64(dk[kt, g]), kk, what=f"{name} L{layer} dk_hat keys")
    sv = check_bf16(f64(dv[kt, g]), kv, what=f"{name} L{layer} dv keys")
    print(f"[full bwd] {name} L{layer}: {len(rows)} rows, {len(keys)} keys; dq {sq['max_err']:.3g} "
          f"dk {sk['max_err']:.3g} dv {sv['max_err']:.3g}", flush=True)
