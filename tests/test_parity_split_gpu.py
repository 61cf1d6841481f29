"""GPU parity of the attention forward's KV split (a work item's key tiles cut
into parts run by separate workgroups and combined per wave in part order).
Forced splits of small cases against the oracle, fused == unfused bitwise
under the split, repeat runs bitwise equal, every output row written, the
automatic split of a grid too small to fill the device, the split policy as a
per-call parameter, a caller workspace reused across shapes, and a split call
captured in a HIP graph."""

import dataclasses

import numpy as np
import pytest
import torch

import decoder_attention_qk_amd as m
import oracle as O
import workloads as W
from gpu_util import bits_f64, check_bf16, check_fp32, dev_bf16, f64, make_case

pytestmark = pytest.mark.gpu

CASES = [
    W.small_workload("split_bshd_b2_s700_g4", num_heads=8, num_kv_heads=2, head_dim=128, batch=2, seqlen=700),
    W.small_workload("split_bshd_s900_g5_w300", num_heads=5, num_kv_heads=1, head_dim=128, seqlen=900,
                     window=300),
    W.small_workload("split_bshd_s520_g1_d64", num_heads=2, num_kv_heads=2, head_dim=64, seqlen=520),
    W.small_workload("split_thd_g3_mixed", num_heads=6, num_kv_heads=2, head_dim=128,
                     segment_lengths=(1, 77, 0, 600, 64, 385)),
    W.small_workload("split_bshd_g16_d64", num_heads=16, num_kv_heads=1, head_dim=64, seqlen=450),
]
IDS = [w.name for w in CASES]
MODES = [2, 3, 8]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.library()


def _with_split(case, mode):
    """The case with the per-call split policy `mode` in its params."""
    case.params = dataclasses.replace(case.params, kv_split=mode)
    return case


@pytest.fixture
def split_mode():
    """split_mode(case, mode): sets the case's per-call KV-split policy."""
    return _with_split


def _sentinel_like(t):
    # bf16 NaN bits: a row the kernel never writes stays NaN
    return torch.full(t.shape, 0x7FC0, dtype=torch.int16, device=t.device).view(torch.bfloat16)


def _q_k_hat(case, layout=None):
    lay = layout if layout is not None else case.layout
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(case.params, lay, case.q, case.k, case.q_gain, case.k_gain,
                                             case.cos, case.sin)
    return q_hat, k_hat


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_split_attention_stage(w, mode, split_mode):
    case = make_case(w)
    q_hat, k_hat = _q_k_hat(case)
    split_mode(case, mode)
    print(f"[split] {w.name} mode {mode}", flush=True)
    o = _sentinel_like(q_hat)
    o, lse = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, o=o, want_lse=True)
    o2, lse2 = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    ro, rl = O.attention(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), case.segs,
                         window=case.x["window"], scaling=case.scaling)
    check_bf16(f64(o), ro, what=f"o split {mode}")
    check_fp32(f64(lse), rl, floor=1.0, what=f"lse split {mode}")
    # a second call reads counters the first left at zero: the same bits
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse, lse2)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_split_fused_core(w, mode, split_mode):
    case = make_case(w)
    split_mode(case, mode)
    print(f"[split fused] {w.name} mode {mode}", flush=True)
    out = _sentinel_like(case.q)
    out, k_hat_f, lse_f = m.muse_attn_core_fwd(case.params, case.layout, case.q, case.k, case.v, case.gate,
                                               case.q_gain, case.k_gain, case.cos, case.sin, out=out,
                                               want_lse=True)
    q_hat, k_hat = _q_k_hat(case)
    o, lse = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    out_u, _ = m.muse_out_norm_gate(case.params, case.layout, o, case.gate)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any()
    ref = O.attn_core(bits_f64(case.x["q"]), bits_f64(case.x["k"]), bits_f64(case.x["v"]),
                      bits_f64(case.x["gate"]), case.segs, **case.oracle_kw())
    check_bf16(f64(out), ref["out"], what=f"fused out split {mode}")
    assert torch.equal(out.view(torch.int16), out_u.view(torch.int16))
    assert torch.equal(lse_f, lse)


def test_split_padded_keys_and_empty_rows(split_mode):
    """Key padding under a split: parts that see only padded keys carry no
    reference; a query with no valid key still gives the zero row."""
    w = W.small_workload("split_pad_b2_s640", num_heads=4, num_kv_heads=1, head_dim=128, batch=2, seqlen=640)
    case = make_case(w)
    valid = np.ones((2, 640), dtype=np.uint8)
    valid[0, :300] = 0          # left padding: the first 300 queries of row 0 see no key
    valid[1, 500:] = 0          # right padding
    valid[1, 64:192] = 0        # two whole padded tiles inside the row
    lay = m.Layout.bshd(2, 640, attention_mask=torch.from_numpy(valid).cuda())
    q_hat, k_hat = _q_k_hat(case, lay)
    split_mode(case, 4)
    o, lse = m.muse_gqa_attn_fwd(case.params, lay, q_hat, k_hat, case.v, want_lse=True)
    out, _, lse_f = m.muse_attn_core_fwd(case.params, lay, case.q, case.k, case.v, case.gate, case.q_gain,
                                         case.k_gain, case.cos, case.sin, want_lse=True)
    out_u, _ = m.muse_out_norm_gate(case.params, lay, o, case.gate)
    torch.cuda.synchronize()
    ro, rl = O.attention(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), case.segs, window=0,
                         scaling=case.scaling, key_valid=valid.reshape(-1))
    check_bf16(f64(o), ro, what="o padded split")
    fin = np.isfinite(rl)
    assert (~fin).any()
    check_fp32(f64(lse)[fin], rl[fin], floor=1.0, what="lse padded split")
    assert torch.isneginf(lse.cpu()[torch.from_numpy(~fin)]).all()
    assert not f64(o)[~fin].any()
    assert torch.equal(out.view(torch.int16), out_u.view(torch.int16))
    assert torch.equal(lse_f, lse)


def test_split_bidirectional(split_mode):
    w = W.small_workload("split_bidir_thd", num_heads=4, num_kv_heads=2, head_dim=128,
                         segment_lengths=(300, 900, 5), use_rope=False)
    case = make_case(w, bidirectional=True)
    q_hat, k_hat = _q_k_hat(case)
    split_mode(case, 3)
    o, lse = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.attention(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), case.segs, window=0,
                         scaling=case.scaling, causal=False)
    check_bf16(f64(o), ro, what="o bidirectional split")
    check_fp32(f64(lse), rl, floor=1.0, what="lse bidirectional split")


def test_automatic_split_of_a_small_grid(split_mode):
    """One KV head of a 2048-token sequence: 64 work items, far fewer than two
    per CU, so the automatic policy splits them; compared with the oracle on
    every element, and with the never-split policy within rounding."""
    w = W.small_workload("split_auto_s2048_h4kv1", num_heads=4, num_kv_heads=1, head_dim=128, seqlen=2048,
                         theta=5.0e5)
    case = make_case(w)
    q_hat, k_hat = _q_k_hat(case)
    assert m.muse_attn_fwd_workspace_size(case.params, case.layout) > 0     # automatic: splits
    o, lse = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    split_mode(case, 1)
    assert m.muse_attn_fwd_workspace_size(case.params, case.layout) == 0
    o1, lse1 = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.attention(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), case.segs, window=0,
                         scaling=case.scaling)
    check_bf16(f64(o), ro, what="o automatic split")
    check_bf16(f64(o1), ro, what="o unsplit")
    check_fp32(f64(lse), rl, floor=1.0, what="lse automatic split")
    # the split reorders sums: the two differ, by rounding only
    assert not torch.equal(o.view(torch.int16), o1.view(torch.int16))
    assert float((lse - lse1).abs().max()) < 1e-5 * max(1.0, float(lse1.abs().max()))


def test_policy_is_per_call():
    """Calls with different policies, interleaved on one stream, each give
    their own policy's bits (no process-wide setting)."""
    w = CASES[0]
    case = make_case(w)
    q_hat, k_hat = _q_k_hat(case)
    p1 = dataclasses.replace(case.params, kv_split=1)
    p3 = dataclasses.replace(case.params, kv_split=3)
    a1, _ = m.muse_gqa_attn_fwd(p1, case.layout, q_hat, k_hat, case.v)
    a3, _ = m.muse_gqa_attn_fwd(p3, case.layout, q_hat, k_hat, case.v)
    b1, _ = m.muse_gqa_attn_fwd(p1, case.layout, q_hat, k_hat, case.v)
    b3, _ = m.muse_gqa_attn_fwd(p3, case.layout, q_hat, k_hat, case.v)
    torch.cuda.synchronize()
    assert torch.equal(a1.view(torch.int16), b1.view(torch.int16))
    assert torch.equal(a3.view(torch.int16), b3.view(torch.int16))
    assert not torch.equal(a1.view(torch.int16), a3.view(torch.int16))


def test_workspace_reused_across_shapes():
    """One caller workspace, filled with garbage, then used by a small split
    call whose slots cover where a larger call's counters sit, then by that
    larger call: each result equals the same call on a fresh workspace (the
    call zeroes its counters itself)."""
    small = make_case(W.small_workload("split_ws_small_s300", num_heads=4, num_kv_heads=1, head_dim=128,
                                       seqlen=300))
    large = make_case(W.small_workload("split_ws_large_b3_s1000", num_heads=8, num_kv_heads=2, head_dim=128,
                                       batch=3, seqlen=1000))
    _with_split(small, 4)
    _with_split(large, 3)
    n_small = m.muse_attn_fwd_workspace_size(small.params, small.layout)
    n_large = m.muse_attn_fwd_workspace_size(large.params, large.layout)
    assert 0 < n_small < n_large
    ws = torch.randint(-128, 127, (n_large,), dtype=torch.int8, device="cuda").view(torch.uint8)
    outs = []
    for case in (small, large, small, large):
        q_hat, k_hat = _q_k_hat(case)
        o_ws, l_ws = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True,
                                         workspace=ws)
        o_new, l_new = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
        outs.append((o_ws, l_ws, o_new, l_new))
    torch.cuda.synchronize()
    for o_ws, l_ws, o_new, l_new in outs:
        assert torch.equal(o_ws.view(torch.int16), o_new.view(torch.int16))
        assert torch.equal(l_ws, l_new)


def test_split_call_in_a_hip_graph():
    """A split forward captured in a graph (its counter reset is a kernel, not
    a memset node) and replayed several times, with eager work and
    synchronisation between replays: every replay equals the eager call."""
    w = CASES[1]
    case = _with_split(make_case(w), 3)
    q_hat, k_hat = _q_k_hat(case)
    ws = torch.empty(m.muse_attn_fwd_workspace_size(case.params, case.layout), dtype=torch.uint8, device="cuda")
    o_ref, lse_ref = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True,
                                         workspace=ws)
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(lse_ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, o=o, lse=lse, workspace=ws,
                                stream=side)
    torch.cuda.synchronize()
    for i in range(4):
        o.zero_()
        lse.zero_()
        junk, _ = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), i
        assert torch.equal(lse, lse_ref), i
    del g


# ---------------------------------------------------------------- backward
# The dQ kernel splits its key tiles as the forward does; the dK/dV kernel
# splits each key block's (query tile, head) steps; each sums its parts' fp32
# accumulators in part order.
BWD_CASES = [CASES[0], CASES[1], CASES[3], CASES[4]]


def _bwd_inputs(case, layout=None):
    lay = layout if layout is not None else case.layout
    q_hat, k_hat = _q_k_hat(case, lay)
    o, lse = m.muse_gqa_attn_fwd(case.params, lay, q_hat, k_hat, case.v, want_lse=True)
    d_o = dev_bf16(W.draw_bf16(tuple(case.q.shape), 1.0, seed=11, workload=case.w.name, layer=0, tensor="d_o"))
    delta = m.muse_attn_bwd_delta(case.params, lay, o, d_o)
    return q_hat, k_hat, o, lse, d_o, delta


@pytest.mark.parametrize("mode", [1, 2, 3, 8])
@pytest.mark.parametrize("w", BWD_CASES, ids=[w.name for w in BWD_CASES])
def test_split_attention_bwd(w, mode, split_mode):
    case = make_case(w)
    q_hat, k_hat, o, lse, d_o, delta = _bwd_inputs(case)
    split_mode(case, mode)
    print(f"[split bwd] {w.name} mode {mode}", flush=True)
    got = m.muse_gqa_attn_bwd(case.params, case.layout, q_hat, k_hat, case.v, d_o, lse, delta)
    again = m.muse_gqa_attn_bwd(case.params, case.layout, q_hat, k_hat, case.v, d_o, lse, delta)
    torch.cuda.synchronize()
    ref = O.attention_bwd(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), f64(d_o), case.segs,
                          window=case.x["window"], scaling=case.scaling, o=f64(o))
    for name, g_, a_, r in zip(("dq_hat", "dk_hat", "dv"), got, again, ref):
        check_bf16(f64(g_), r, what=f"{name} split {mode}")
        assert torch.equal(g_.view(torch.int16), a_.view(torch.int16)), name


def test_split_attention_bwd_padded_keys(split_mode):
    w = W.small_workload("split_bwd_pad_b2_s640", num_heads=8, num_kv_heads=2, head_dim=128, batch=2, seqlen=640)
    case = make_case(w)
    valid = np.ones((2, 640), dtype=np.uint8)
    valid[0, :300] = 0
    valid[1, 64:192] = 0
    valid[1, 500:] = 0
    lay = m.Layout.bshd(2, 640, attention_mask=torch.from_numpy(valid).cuda())
    q_hat, k_hat, o, lse, d_o, delta = _bwd_inputs(case, lay)
    split_mode(case, 4)
    dq, dk, dv = m.muse_gqa_attn_bwd(case.params, lay, q_hat, k_hat, case.v, d_o, lse, delta)
    torch.cuda.synchronize()
    rq, rk, rv = O.attention_bwd(f64(q_hat), f64(k_hat), bits_f64(case.x["v"]), f64(d_o), case.segs, window=0,
                                 scaling=case.scaling, o=f64(o), key_valid=valid.reshape(-1).astype(bool))
    check_bf16(f64(dq), rq, what="dq_hat padded split")
    check_bf16(f64(dk), rk, what="dk_hat padded split")
    check_bf16(f64(dv), rv, what="dv padded split")
    flat = torch.from_numpy(valid.reshape(-1) == 0).cuda()
    assert torch.all(dk[flat] == 0) and torch.all(dv[flat] == 0)


def test_split_on_a_side_stream_matches_the_default_stream(split_mode):
    """A call on a torch side stream (non-blocking) zeroes its counters in
    its own stream order: it equals the default stream's call."""
    w = W.small_workload("split_side_stream_s1100", num_heads=8, num_kv_heads=2, head_dim=128, seqlen=1100)
    case = make_case(w)
    q_hat, k_hat = _q_k_hat(case)
    split_mode(case, 3)
    o_ref, lse_ref = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o, lse = m.muse_gqa_attn_fwd(case.params, case.layout, q_hat, k_hat, case.v, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, lse_ref)
