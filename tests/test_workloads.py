"""The seeded workload generator: shapes, determinism and the packed lengths."""

import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_thd_lengths_match_fixture():
    with open(os.path.join(GOLDEN, "thd_lengths.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    expected = tuple(int(x) for x in rows[0].split())
    assert W.thd_lengths(0) == expected
    w = W.WORKLOADS["thd_16seg_h40kv8_d128"]
    assert w.tokens == 68143 and w.max_seqlen == 7960
    cu = w.cu_seqlens()
    assert cu.dtype == np.int32 and cu[0] == 0 and cu[-1] == 68143 and len(cu) == 17


def test_inputs_are_seeded_and_shaped():
    w = W.small_workload("t", num_heads=4, num_kv_heads=2, head_dim=64, batch=2, seqlen=33)
    a = W.make_layer_inputs(w)
    b = W.make_layer_inputs(w)
    for key in ("q", "k", "v", "gate", "q_gain", "k_gain"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["q"].shape == (66, 4, 64) and a["q"].dtype == np.uint16
    assert a["k"].shape == (66, 2, 64) and a["v"].shape == (66, 2, 64)
    assert a["q_gain"].dtype == np.float32 and a["q_gain"].shape == (64,)
    assert not np.array_equal(a["q"][:, :2], a["k"])       # independent streams
    # gains are bf16-representable float32 values
    g = a["q_gain"].view(np.uint32)
    assert np.all((g & 0xFFFF) == 0)


def test_value_distribution_matches_std():
    w = W.WORKLOADS["bshd_1x128_h4kv1_d64"]
    x = W.make_layer_inputs(w)
    q = (x["q"].astype(np.uint32) << 16).view(np.float32)
    assert abs(q.std() - 1.0) < 0.02 and abs(q.mean()) < 0.02
    g = x["q_gain"]
    assert 0.02 < g.std() < 0.08


def test_mix_workload_layers():
    w = W.WORKLOADS["bshd_1x32768_h64kv8_d128_mix"]
    assert w.layers == ((8192, True), (8192, True), (8192, True), (0, False))
    assert w.gate_std == 4.0 and w.tokens == 32768
