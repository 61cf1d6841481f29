"""Parity of the whole path on seeded random configurations (GPU).

Each case draws, from its own seed, one configuration the fixed cases do not
enumerate: head dim 64 or 128, 1-3 KV heads with a group of 1-8 query heads,
BSHD (1-3 rows of 1-1500 tokens) or packed THD (1-6 documents of 0-1500
tokens, some of length 1), a window (none, or 1 up to past the longest row),
RoPE on or off in either rotation mode, query_scale 1 or 0.75, the
bidirectional mask, key padding, explicit position_ids, and the KV-split policy
(automatic, never, 2, 3 or 8 parts).  Checked against the oracle, with the bars
of the other parity tests:
* the fused core's output: the row bar and the elementwise bar;
* the attention backward on the GPU's own q_hat/k_hat: the row bar on dq_hat,
  dk_hat and dv;
* every third case, the whole core backward from the raw inputs: dv and dgate
  by the row bar, dq, dk and the gain gradients against the same backward
  carried out on magnitudes (their sums cancel).
"""

import dataclasses

import numpy as np
import pytest
import torch

import decoder_attention_qk_amd as m
import oracle as O
import workloads as W
from gpu_util import (bits_f64, check_bf16, check_scaled, core_bwd_magnitudes, dev_bf16, f64, make_case)

pytestmark = pytest.mark.gpu

SEEDS = list(range(5000, 5060))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.library()


def _draw_config(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128], p=[0.3, 0.7]))
    hkv = int(rng.integers(1, 4))
    hq = hkv * int(rng.integers(1, 9))
    thd = bool(rng.random() < 0.4)
    bidir = bool(rng.random() < 0.15)
    if thd:
        nseg = int(rng.integers(1, 7))
        lens = [int(x) for x in rng.integers(0, 1500 if rng.random() < 0.3 else 600, nseg)]
        if rng.random() < 0.3:
            lens[int(rng.integers(0, nseg))] = 1
        if sum(lens) == 0:
            lens[0] = 5
        batch, seqlen, maxlen = 0, 0, max(lens)
    else:
        lens = []
        batch = int(rng.integers(1, 4))
        seqlen = int(rng.integers(1, 1500 if rng.random() < 0.3 else 700))
        maxlen = seqlen
    cfg = dict(seed=seed, d=d, hq=hq, hkv=hkv, thd=thd, lens=lens, batch=batch, seqlen=seqlen, bidir=bidir)
    cfg["window"] = 0 if (bidir or rng.random() < 0.5) else int(rng.integers(1, maxlen + 2))
    cfg["use_rope"] = bool(rng.random() < 0.8)
    cfg["upcast"] = bool(rng.random() < 0.8)
    cfg["query_scale"] = 0.75 if rng.random() < 0.2 else 1.0
    cfg["split"] = int(rng.choice([0, 1, 2, 3, 8]))
    cfg["pad"] = (not thd) and (not bidir) and bool(rng.random() < 0.3)
    cfg["posids"] = (not thd) and (not cfg["pad"]) and cfg["use_rope"] and bool(rng.random() < 0.25)
    return cfg, rng


def _pad_mask(rng, batch, seqlen):
    valid = np.ones((batch, seqlen), dtype=bool)
    for b in range(batch):
        kind = int(rng.integers(0, 3))
        if kind == 0 and seqlen > 1:
            valid[b, seqlen - int(rng.integers(1, seqlen)):] = False
        elif kind == 1 and seqlen > 1:
            valid[b, :int(rng.integers(1, seqlen))] = False
        else:
            valid[b] = rng.random(seqlen) > 0.35
    return valid


@pytest.mark.parametrize("seed", SEEDS)
def test_random_configuration(seed):
    cfg, rng = _draw_config(seed)
    print(f"[random parity] {cfg}", flush=True)
    name = f"rand{seed}"
    w = W.small_workload(name, num_heads=cfg["hq"], num_kv_heads=cfg["hkv"], head_dim=cfg["d"],
                         batch=cfg["batch"], seqlen=cfg["seqlen"], segment_lengths=cfg["lens"],
                         window=cfg["window"], use_rope=cfg["use_rope"],
                         theta=1.0e4 if cfg["d"] == 64 else 5.0e5, seed=seed)
    case = make_case(w, query_scale=cfg["query_scale"], upcast_rope=cfg["upcast"], bidirectional=cfg["bidir"])
    case.params = dataclasses.replace(case.params, kv_split=cfg["split"])
    kw = case.oracle_kw()
    lay, cos, sin, key_valid = case.layout, case.cos, case.sin, None
    if cfg["pad"]:
        valid = _pad_mask(rng, cfg["batch"], cfg["seqlen"])
        lay = m.Layout.bshd(cfg["batch"], cfg["seqlen"], attention_mask=torch.from_numpy(valid).cuda())
        key_valid = valid.reshape(-1)
    if cfg["posids"]:
        pos = rng.integers(0, 4096, cfg["batch"] * cfg["seqlen"]).astype(np.int32)
        cos, sin = m.muse_rope_cos_sin(w.theta, cfg["d"], 4096)
        lay = m.Layout.bshd(cfg["batch"], cfg["seqlen"], position_ids=torch.from_numpy(pos).cuda())
        kw["position_ids"] = pos

    # the fused core, against the oracle's whole forward
    out, _, _ = m.muse_attn_core_fwd(case.params, lay, case.q, case.k, case.v, case.gate, case.q_gain,
                                     case.k_gain, cos, sin)
    torch.cuda.synchronize()
    ref = O.attn_core(bits_f64(case.x["q"]), bits_f64(case.x["k"]), bits_f64(case.x["v"]),
                      bits_f64(case.x["gate"]), case.segs, key_valid=key_valid, **kw)
    check_bf16(f64(out), ref["out"], what=f"random {seed} fused out")

    # the attention backward on the GPU's own q_hat/k_hat
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, lay, case.q, case.k, case.q_gain, case.k_gain, cos, sin)
    o, lse = m.muse_gqa_attn_fwd(case.params, lay, q_hat, k_hat, case.v, want_lse=True)
    d_o = dev_bf16(W.draw_bf16(tuple(case.q.shape), 1.0, seed=7, workload=name, layer=0, tensor="d_o"))
    delta = m.muse_attn_bwd_delta(case.params, lay, o, d_o)
    dq, dk, dv = m.muse_gqa_attn_bwd(case.params, lay, q_hat, k_hat, case.v, d_o, lse, delta)
    torch.cuda.synchronize()
    rq, rk, rv = O.attention_bwd(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), f64(d_o), case.segs,
                                 window=case.x["window"], scaling=case.scaling, o=f64(o),
                                 causal=not cfg["bidir"], key_valid=key_valid)
    for got, want, what in ((dq, rq, "dq_hat"), (dk, rk, "dk_hat"), (dv, rv, "dv")):
        check_bf16(f64(got), want, what=f"random {seed} {what}", elem_tol=None)

    # every third case: the whole core backward from the raw inputs
    if seed % 3 == 0 and not cfg["pad"]:
        dout_bits = W.draw_bf16(tuple(case.q.shape), 1.0, seed=3, workload=name, layer=0, tensor="dout")
        grads = m.muse_attn_core_bwd(case.params, lay, case.q, case.k, case.v, case.gate, dev_bf16(dout_bits),
                                     case.q_gain, case.k_gain, cos, sin)
        torch.cuda.synchronize()
        gq, gk, gv, gg, gqg, gkg = grads
        args = (bits_f64(case.x["q"]), bits_f64(case.x["k"]), bits_f64(case.x["v"]), bits_f64(case.x["gate"]))
        dout = O.bf16_bits_to_f64(dout_bits)
        rb = O.attn_core_bwd(*args, dout, case.segs, **kw)
        mag = core_bwd_magnitudes(case, dout, rb, kw)
        check_bf16(f64(gv), rb["dv"], what=f"random {seed} core dv", elem_tol=None)
        check_bf16(f64(gg), rb["dgate"], what=f"random {seed} core dgate", elem_tol=None)
        check_scaled(f64(gq), rb["dq"], mag["dq"], f"random {seed} core dq")
        check_scaled(f64(gk), rb["dk"], mag["dk"], f"random {seed} core dk")
        check_scaled(f64(gqg)[None], rb["dq_gain"][None], mag["dq_gain"][None], f"random {seed} core dq_gain")
        check_scaled(f64(gkg)[None], rb["dk_gain"][None], mag["dk_gain"][None], f"random {seed} core dk_gain")
