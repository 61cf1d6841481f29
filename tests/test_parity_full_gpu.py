"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (the fused core), checked against the oracle on sampled rows: one row
of every attention work item (segment, block of query tokens, KV head), every
segment's first/last rows, rows around each window edge and random rows over
all heads (the sequences past 32k: all but the work-item rows).  The
normalised keys (a full output) are checked everywhere."""

import numpy as np
import pytest
import torch

import decoder_attention_qk_amd as m
import oracle as O
import workloads as W
from gpu_util import bits_f64, check_bf16, check_fp32, f64, make_case, sample_rows

pytestmark = pytest.mark.gpu

FULL = [
    ("bshd_1x128_h4kv1_d64", 0),
    ("bshd_2x4096_h32kv8_d128", 0),
    ("bshd_1x16384_h32kv8_d128_w4096", 0),
    ("thd_16seg_h40kv8_d128", 0),
    ("bshd_1x32768_h64kv8_d128_mix", 0),
    ("bshd_1x32768_h64kv8_d128_mix", 1),
    ("bshd_1x32768_h64kv8_d128_mix", 2),
    ("bshd_1x32768_h64kv8_d128_mix", 3),
    # one GPU's share of the head-sharded layers (the 2x4096 share takes the KV split)
    ("bshd_2x4096_h4kv1_d128", 0),
    ("bshd_1x16384_h4kv1_d128_w4096", 0),
    ("thd_16seg_h5kv1_d128", 0),
    ("bshd_1x32768_h8kv1_d128_mix", 3),
]


# sequences past the configurations' 32k: positions, window bounds, table rows
# and tile offsets at their largest values
LONG = {
    "bshd_1x131072_h8kv1_d128": W.small_workload("bshd_1x131072_h8kv1_d128", num_heads=8, num_kv_heads=1,
                                                 head_dim=128, seqlen=131072, theta=5.0e5),
    "thd_2seg_long_h8kv2_d128_w70000": W.small_workload("thd_2seg_long_h8kv2_d128_w70000", num_heads=8,
                                                        num_kv_heads=2, head_dim=128,
                                                        segment_lengths=(100000, 31072), window=70000,
                                                        theta=5.0e5),
}
FULL += [(n, 0) for n in LONG]


@pytest.mark.parametrize("name,layer", FULL, ids=[f"{n}-L{l}" for n, l in FULL])
def test_full_size_sampled_rows(name, layer):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = LONG[name] if name in LONG else W.WORKLOADS[name]
    print(f"[full] {name} layer {layer}", flush=True)
    case = make_case(w, layer)
    out, k_hat, lse = m.muse_attn_core_fwd(case.params, case.layout, case.q, case.k, case.v,
                                           case.gate, case.q_gain, case.k_gain, case.cos, case.sin,
                                           want_lse=True)
    torch.cuda.synchronize()
    rows = sample_rows(case.segs, w.num_heads, case.x["window"], n_random=192, seed=layer,
                       num_kv_heads=None if name in LONG else w.num_kv_heads)
    tok = np.array([t for t, _ in rows])
    hd = np.array([h for _, h in rows])
    kw = case.oracle_kw()
    ref = O.attn_core_rows(bits_f64(case.x["q"][tok, hd]), bits_f64(case.x["k"]),
                           bits_f64(case.x["v"]), bits_f64(case.x["gate"][tok, hd]), case.segs,
                           rows, num_heads=w.num_heads, grouped=True, **kw)
    ti, hi = torch.from_numpy(tok).cuda(), torch.from_numpy(hd).cuda()
    st = check_bf16(f64(out[ti, hi]), ref["out"], what=f"{name} L{layer} out rows")
    sk = check_bf16(f64(k_hat), ref["k_hat"], what=f"{name} L{layer} k_hat")
    assert sk["exact"] > 0.999, sk
    # lse (an FP32 intermediate) against the oracle fed the GPU's own q_hat/k_hat
    q_hat, _, _, _ = m.muse_qk_norm_rope(case.params, case.layout, case.q, None, case.q_gain, None,
                                         case.cos, case.sin)
    torch.cuda.synchronize()
    _, rl = O.attention_rows_grouped(f64(q_hat[ti, hi]), f64(k_hat), bits_f64(case.x["v"]), case.segs, rows,
                                     num_heads=w.num_heads, window=case.x["window"], scaling=case.scaling)
    check_fp32(f64(lse[ti, hi]), rl, floor=1.0, what=f"{name} L{layer} lse rows")
    del q_hat
    print(f"[full] {name} L{layer}: {len(rows)} rows, out row err {st['max_err']:.4f}, "
          f"elem err {st['elem_err']:.4f}", flush=True)
