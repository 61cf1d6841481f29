"""The allocation-free entry point muse_qk_norm_rope_bwd_static (for callers
that cannot allocate: code under graph capture, tight serving loops): called
through the C ABI, it must give the bits of muse_qk_norm_rope_bwd with a
caller workspace, on two calls in a row, the second with a smaller input (the
library-held scratch keeps the first call's partial sums, which the second
must overwrite)."""

import ctypes

import numpy as np
import pytest
import torch

import decoder_attention_qk_amd as m
import workloads as W
from gpu_util import dev_bf16, make_case

pytestmark = pytest.mark.gpu

CASES = [
    W.small_workload("noalloc_thd_big", num_heads=8, num_kv_heads=2, head_dim=128,
                     segment_lengths=(700, 1, 333, 1200), theta=5.0e5),
    W.small_workload("noalloc_bshd_small", num_heads=4, num_kv_heads=1, head_dim=64, batch=2, seqlen=45),
]


def _p(t):
    return None if t is None else t.data_ptr()


def _static_call(case, dqh, dkh, dq, dk, dqg, dkg):
    lib = m.library()
    fn = lib.muse_qk_norm_rope_bwd_static
    p, l = case.params.to_c(), case.layout.to_c()
    n_pos = case.cos.shape[0] if case.cos is not None else 0
    st = fn(ctypes.byref(p), ctypes.byref(l), _p(case.q), _p(case.k), _p(case.q_gain), _p(case.k_gain),
            _p(case.cos), _p(case.sin), n_pos, _p(dqh), _p(dkh), _p(dq), _p(dk), _p(dqg), _p(dkg),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.muse_last_error().decode()


def test_static_scratch_matches_the_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fn = m.library().muse_qk_norm_rope_bwd_static
    fn.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int32] + [ctypes.c_void_p] * 7
    fn.restype = ctypes.c_int
    for i, w in enumerate(CASES):          # the second case is smaller
        case = make_case(w, query_scale=0.75)
        print(f"[noalloc] {w.name}", flush=True)
        dqh = dev_bf16(W.draw_bf16(tuple(case.q.shape), 1.0, seed=5, workload=w.name, layer=0, tensor="dqh"))
        dkh = dev_bf16(W.draw_bf16(tuple(case.k.shape), 1.0, seed=6, workload=w.name, layer=0, tensor="dkh"))
        ref = m.muse_qk_norm_rope_bwd(case.params, case.layout, case.q, case.k, case.q_gain, case.k_gain,
                                      case.cos, case.sin, dqh, dkh)
        outs = (torch.empty_like(case.q), torch.empty_like(case.k), torch.empty_like(case.q_gain),
                torch.empty_like(case.k_gain))
        for o in outs:
            o.fill_(float("nan"))
        _static_call(case, dqh, dkh, *outs)
        torch.cuda.synchronize()
        for name, got, want in zip(("dq", "dk", "dq_gain", "dk_gain"), outs, ref):
            assert torch.equal(got.view(torch.int32) if got.dtype == torch.float32 else got.view(torch.int16),
                               want.view(torch.int32) if want.dtype == torch.float32 else want.view(torch.int16)), \
                (w.name, name)
