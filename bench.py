"""Benchmark of the Muse Spark Open attention core on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
for each layer of the workload the key norm/RoPE pass (the first rotating
layer's pass also builds the FP32 RoPE table, in the same launch) and the
fused attention kernel (query norm/RoPE prologue, causal GQA flash attention,
output norm x sigmoid gate epilogue).  Inputs are resident in
HBM before the timed region.  Prints one JSON line.  Besides the step it
reports the unfused stages (flushed caches) and the backward entry points of
layer 0 (--no-stages, --no-backward skip them).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "attention TFLOP/s (causal-adjusted) + norm/RoPE/gate GB/s, % of roofline"
DEFAULT_WORKLOAD = "bshd_2x4096_h32kv8_d128"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
EVENT_EVERY = 4                # timed steps between two steps with per-launch events
EPS = 1e-6


def visible_pairs(length: int, window: int) -> int:
    """Exact count of visible (query, key) pairs in one causal sequence."""
    if window <= 0 or window >= length:
        return length * (length + 1) // 2
    return window * (window + 1) // 2 + (length - window) * window


def seq_lengths(w: W.Workload) -> list[int]:
    return list(w.segment_lengths) if w.is_thd else [w.seqlen] * w.batch


def layer_flop(w: W.Workload, window: int) -> int:
    return 4 * w.head_dim * w.num_heads * sum(visible_pairs(n, window) for n in seq_lengths(w))


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU raises its clocks over the first ~30 ms of sustained work, so the
    # default warmup runs 100 steps before the timed region
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(W.WORKLOADS))
    ap.add_argument("--kv-split", type=int, default=0,
                    help="attention KV-split policy: 0 automatic, 1 never, n >= 2 n parts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true", help="skip the per-stage (unfused) measurements")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurements")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (reference kernel for HBM counters)")
    return ap.parse_args()


def kernel_source_digest() -> str:
    """Digest of the sources the fused attention kernel is built from: its
    own file, the two device headers it includes, and its argument struct
    (the rest of kernels.hpp declares other kernels)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decoder_attention_qk_amd", "csrc")
    for name in ("attn_fwd.hip", "attn_common.hpp", "device_common.hpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(csrc, "kernels.hpp")) as f:
        text = f.read()
    start = text.index("struct AttnArgs {")
    h.update(text[start:text.index("};", start)].encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, launches: int):
    """HBM bytes per launch of the fused attention kernel from the committed
    rocprofv3 counter summary, or None when it was taken on other sources."""
    path = os.path.join(ROOT, "profiles", f"attn_fused_traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    return int(rec["fetch_bytes_per_launch"]) + int(rec["write_bytes_per_launch"])


class Bench:
    def __init__(self, w: W.Workload):
        import torch

        import decoder_attention_qk_amd as m
        self.torch, self.m, self.w = torch, m, w
        dev = torch.device("cuda:0")
        self.dev = dev

        def bf(a):
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

        self.layers = []
        for li in range(len(w.layers)):
            x = W.make_layer_inputs(w, li)
            p = m.AttnParams(head_dim=w.head_dim, num_heads=w.num_heads,
                             num_key_value_heads=w.num_kv_heads, sliding_window=x["window"],
                             use_rope=x["use_rope"], scaling=float(np.float32(w.head_dim ** -0.5)),
                             qk_eps=EPS, out_eps=EPS)
            t = dict(params=p, q=bf(x["q"]), k=bf(x["k"]), v=bf(x["v"]), gate=bf(x["gate"]),
                     q_gain=torch.from_numpy(x["q_gain"]).to(dev),
                     k_gain=torch.from_numpy(x["k_gain"]).to(dev), window=x["window"])
            t["k_hat"] = torch.empty_like(t["k"])
            t["out"] = torch.empty_like(t["q"])
            self.layers.append(t)
        if w.is_thd:
            cu = torch.from_numpy(w.cu_seqlens()).to(dev)
            self.layout = m.Layout.thd(cu, w.max_seqlen, total_tokens=w.tokens)
        else:
            self.layout = m.Layout.bshd(w.batch, w.seqlen)
        self.n_pos = max(1, w.max_seqlen)
        self.cos = torch.empty((self.n_pos, w.head_dim // 2), dtype=torch.float32, device=dev)
        self.sin = torch.empty_like(self.cos)
        torch.cuda.synchronize()

    def step(self, ev=None):
        """One pass of the hot path; optionally records events around each launch.
        The first rotating layer's key pass also builds the RoPE table (one
        launch); later layers read it."""
        m = self.m
        if ev is not None:
            ev[0].record()
        table_built = False
        for li, t in enumerate(self.layers):
            cos, sin = (self.cos, self.sin) if t["params"].use_rope else (None, None)
            if ev is not None:
                ev[1 + 3 * li].record()
            if t["params"].use_rope and not table_built:
                m.muse_qk_norm_rope_table(t["params"], self.layout, None, t["k"], None, t["k_gain"],
                                          theta=self.w.theta, n_pos=self.n_pos, cos_out=self.cos,
                                          sin_out=self.sin, k_out=t["k_hat"])
                table_built = True
            else:
                m.muse_qk_norm_rope(t["params"], self.layout, None, t["k"], None, t["k_gain"], cos, sin,
                                    k_out=t["k_hat"])
            if ev is not None:
                ev[2 + 3 * li].record()
            m.muse_attn_fused_fwd(t["params"], self.layout, t["q"], t["k_hat"], t["v"], t["gate"],
                                  t["q_gain"], cos, sin, out=t["out"])
            if ev is not None:
                ev[3 + 3 * li].record()

    def n_events(self):
        return 1 + 3 * len(self.layers)


def measure_stages(b: Bench, iters: int = 5) -> dict:
    """Unfused stages, each timed alone after reading a 512 MiB buffer, which
    refills the 256 MB Infinity Cache with clean unrelated lines, so the
    HBM-bound kernels are charged HBM traffic (a write-based flush would leave
    dirty lines for the measured kernel to write back)."""
    torch, m, w = b.torch, b.m, b.w
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=b.dev)
    t = b.layers[0]
    cos, sin = (b.cos, b.sin) if t["params"].use_rope else (None, None)
    q_hat, k_hat = torch.empty_like(t["q"]), torch.empty_like(t["k"])
    o = torch.empty_like(t["q"])
    out = torch.empty_like(t["q"])

    def timed(fn):
        ts = []
        for _ in range(iters + 1):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts[1:]))

    qb = t["q"].numel() * 2
    kb = t["k"].numel() * 2
    res = {}
    s = timed(lambda: m.muse_qk_norm_rope(t["params"], b.layout, t["q"], t["k"], t["q_gain"], t["k_gain"],
                                          cos, sin, q_out=q_hat, k_out=k_hat))
    res["qk_norm_rope"] = dict(us=s * 1e6, GBps=2 * (qb + kb) / s / 1e9)
    s = timed(lambda: m.muse_gqa_attn_fwd(t["params"], b.layout, q_hat, k_hat, t["v"], o=o))
    res["gqa_attn_fwd"] = dict(us=s * 1e6, TFLOPs=layer_flop(w, t["window"]) / s / 1e12)
    s = timed(lambda: m.muse_out_norm_gate(t["params"], b.layout, o, t["gate"], out=out))
    res["out_norm_gate"] = dict(us=s * 1e6, GBps=3 * qb / s / 1e9)
    s = timed(lambda: m.muse_qk_norm_rope(t["params"], b.layout, None, t["k"], None, t["k_gain"], cos, sin,
                                          k_out=k_hat))
    res["k_norm_rope"] = dict(us=s * 1e6, GBps=2 * kb / s / 1e9)
    s = timed(lambda: m.muse_attn_fused_fwd(t["params"], b.layout, t["q"], k_hat, t["v"], t["gate"],
                                            t["q_gain"], cos, sin, out=out))
    res["attn_fused_fwd_flushed"] = dict(us=s * 1e6, TFLOPs=layer_flop(w, t["window"]) / s / 1e12)
    for v in res.values():
        if "GBps" in v:
            v["frac_hbm"] = v["GBps"] / PEAK_HBM_GBPS
        if "TFLOPs" in v:
            v["frac_mfma"] = v["TFLOPs"] / PEAK_BF16_TFLOPS
        for key in list(v):
            v[key] = round(v[key], 4)
    del flush
    return res


def measure_backward(b: Bench, warmup: int = 20, iters: int = 50) -> dict:
    """The backward of layer 0 (warm clocks, back-to-back launches, events
    around each entry point): output norm/gate backward, attention backward
    (dQ kernel + dK/dV kernel), Q/K norm/RoPE backward, and the whole
    muse_attn_core_bwd with the forward's O and LSE given.  Attention FLOP
    are algorithmic: five products of 2 D flop per visible (query, key, head)
    -- 2.5x the forward's -- although the kernels recompute S and dP once more."""
    torch, m, w = b.torch, b.m, b.w
    t = b.layers[0]
    p, lay = t["params"], b.layout
    cos, sin = (b.cos, b.sin) if p.use_rope else (None, None)
    m.muse_rope_cos_sin(w.theta, w.head_dim, b.n_pos, b.cos, b.sin)
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(p, lay, t["q"], t["k"], t["q_gain"], t["k_gain"], cos, sin)
    o, lse = m.muse_gqa_attn_fwd(p, lay, q_hat, k_hat, t["v"], want_lse=True)
    g = torch.Generator(device=b.dev)
    g.manual_seed(7)
    dout = torch.randn(t["q"].shape, generator=g, device=b.dev).to(torch.bfloat16)
    d_o, dgate, delta = m.muse_out_norm_gate_bwd(p, lay, o, t["gate"], dout)
    dq_hat, dk_hat, dv = m.muse_gqa_attn_bwd(p, lay, q_hat, k_hat, t["v"], d_o, lse, delta)
    dq, dk, dqg, dkg = m.muse_qk_norm_rope_bwd(p, lay, t["q"], t["k"], t["q_gain"], t["k_gain"], cos, sin,
                                               dq_hat, dk_hat)
    res_core = m.muse_attn_core_bwd(p, lay, t["q"], t["k"], t["v"], t["gate"], dout, t["q_gain"], t["k_gain"],
                                    cos, sin, o=o, lse=lse)
    size = ctypes.c_size_t(0)
    pc, lc = p.to_c(), lay.to_c()
    m.library().muse_attn_core_bwd_workspace_size(ctypes.byref(pc), ctypes.byref(lc), ctypes.byref(size))
    ws = torch.empty(size.value, dtype=torch.uint8, device=b.dev)
    calls = [
        lambda: m.muse_out_norm_gate_bwd(p, lay, o, t["gate"], dout, d_o=d_o, dgate=dgate, delta=delta),
        lambda: m.muse_gqa_attn_bwd(p, lay, q_hat, k_hat, t["v"], d_o, lse, delta, dq_hat=dq_hat,
                                    dk_hat=dk_hat, dv=dv),
        lambda: m.muse_qk_norm_rope_bwd(p, lay, t["q"], t["k"], t["q_gain"], t["k_gain"], cos, sin, dq_hat,
                                        dk_hat, dq=dq, dk=dk, dq_gain=dqg, dk_gain=dkg),
        lambda: m.muse_attn_core_bwd(p, lay, t["q"], t["k"], t["v"], t["gate"], dout, t["q_gain"],
                                     t["k_gain"], cos, sin, o=o, lse=lse, dq=res_core[0], dk=res_core[1],
                                     dv=res_core[2], dgate=res_core[3], dq_gain=res_core[4],
                                     dk_gain=res_core[5], workspace=ws),
    ]
    for _ in range(warmup):
        for c in calls:
            c()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(iters)]
    for i in range(iters):
        evs[i][0].record()
        for j, c in enumerate(calls):
            c()
            evs[i][j + 1].record()
    torch.cuda.synchronize()
    us = [float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(iters)])) * 1e3
          for j in range(len(calls))]
    qb, kb = t["q"].numel() * 2, t["k"].numel() * 2
    flop = 2.5 * layer_flop(w, t["window"])
    return {
        "out_norm_gate_bwd": {"us": round(us[0], 2), "GBps": round(5 * qb / us[0] / 1e3, 1),
                              "frac_hbm": round(5 * qb / us[0] / 1e3 / PEAK_HBM_GBPS, 4)},
        "gqa_attn_bwd": {"us": round(us[1], 2), "TFLOPs": round(flop / us[1] / 1e6, 2),
                         "frac_mfma": round(flop / us[1] / 1e6 / PEAK_BF16_TFLOPS, 4),
                         "flop_algorithmic": int(flop)},
        "qk_norm_rope_bwd": {"us": round(us[2], 2), "GBps": round(3 * (qb + kb) / us[2] / 1e3, 1),
                             "frac_hbm": round(3 * (qb + kb) / us[2] / 1e3 / PEAK_HBM_GBPS, 4)},
        "attn_core_bwd": {"us": round(us[3], 2), "TFLOPs": round(flop / us[3] / 1e6, 2)},
    }


def cpu_baseline(w: W.Workload, budget_s: float = 12.0) -> dict:
    """The FP64 oracle, as it stands, on whole (sequence, KV group) units of
    the same workload until about `budget_s` seconds of CPU work are done."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas")
    except Exception:
        threads = 0
    threads = threads or 1
    x = W.make_layer_inputs(w, 0)
    window, use_rope = x["window"], x["use_rope"]
    g = w.num_heads // w.num_kv_heads
    starts = np.concatenate([[0], np.cumsum(seq_lengths(w))])[:-1]
    units = [(int(s), int(n), kv) for s, n in zip(starts, seq_lengths(w)) for kv in range(w.num_kv_heads)]
    units.sort(key=lambda u: -u[1])
    flop = 0
    done = 0
    t0 = time.perf_counter()
    for s0, n, kv in units:
        sl = slice(s0, s0 + n)
        hs = slice(kv * g, (kv + 1) * g)
        O.attn_core(O.bf16_bits_to_f64(x["q"][sl, hs]), O.bf16_bits_to_f64(x["k"][sl, kv:kv + 1]),
                    O.bf16_bits_to_f64(x["v"][sl, kv:kv + 1]), O.bf16_bits_to_f64(x["gate"][sl, hs]),
                    O.Segments.bshd(1, n), theta=w.theta, eps=EPS, out_eps=EPS,
                    scaling=float(np.float32(w.head_dim ** -0.5)), window=window, use_rope=use_rope,
                    q_gain=x["q_gain"].astype(np.float64), k_gain=x["k_gain"].astype(np.float64))
        flop += 4 * w.head_dim * g * visible_pairs(n, window)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(flop / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {len(units)} (sequence, kv-group) units of layer 0 ({g} query heads each), "
                      f"full oracle path (norm, RoPE, attention, norm-gate) in {el:.1f} s; "
                      f"BLAS threads {threads}, elementwise numpy single-threaded"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): the library has no "
              "multi-GPU path; each GPU would run it on its own share of the KV heads", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    import decoder_attention_qk_amd as m
    w = W.WORKLOADS[args.workload]
    m.muse_attn_set_kv_split(args.kv_split)
    b = Bench(w)
    if args.calibrate_copy:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=b.dev)   # 256 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        b.step()
    torch.cuda.synchronize()

    # Per-launch events on every EVENT_EVERY-th timed step only: each timed
    # event is a marker packet between dependent kernels, and four of them
    # per step add ~13 us (4 %) to the step; sampled steps keep the kernel
    # timing live inside the timed region at ~1 % cost.
    sampled = list(range(0, args.steps, EVENT_EVERY))
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(b.n_events())] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        b.step(evs.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    nl = len(b.layers)
    attn_s = np.array([[evs[i][2 + 3 * li].elapsed_time(evs[i][3 + 3 * li]) * 1e-3 for li in range(nl)]
                       for i in sampled])
    kpass_s = np.array([[evs[i][1 + 3 * li].elapsed_time(evs[i][2 + 3 * li]) * 1e-3 for li in range(nl)]
                        for i in sampled])
    flop_layers = [layer_flop(w, t["window"]) for t in b.layers]
    flop_step = sum(flop_layers)
    step_s = wall / args.steps
    # dominant kernel: the fused attention kernel; achieved = algorithmic flop
    # per launch / mean launch duration, over all its launches in the timed region
    achieved = float(np.mean([flop_layers[li] / attn_s[:, li].mean() for li in range(nl)])) / 1e12
    kb = b.layers[0]["k"].numel() * 2
    qb = b.layers[0]["q"].numel() * 2
    line = {
        "metric": METRIC,
        "value": round(flop_step / step_s / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "tokens": w.tokens, "batch": w.batch if not w.is_thd else 1,
            "seq_len": w.max_seqlen, "segments": len(seq_lengths(w)), "num_heads": w.num_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "layers": [{"sliding_window": t["window"], "use_rope": bool(t["params"].use_rope)} for t in b.layers],
            "flop_per_step_causal": flop_step,
            "share_of": W.SHARE_OF.get(w.name),
            "kv_split_policy": args.kv_split,
        },
        "roofline": {
            "bound": "mfma", "kernel": "attn_fwd_kernel<128,fused>" if w.head_dim == 128 else "attn_fwd_kernel<64,fused>",
            "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(w.name, nl),
            "launch_us": round(float(attn_s.mean()) * 1e6, 2),
        },
        "k_norm_rope": {
            "launch_us": round(float(kpass_s.mean()) * 1e6, 2),
            "GBps": round(2 * kb / float(kpass_s.mean()) / 1e9, 1),
            "frac_hbm": round(2 * kb / float(kpass_s.mean()) / 1e9 / PEAK_HBM_GBPS, 4),
        },
        "fused_bytes_per_layer": 3 * qb + 2 * kb,
    }
    if not args.no_stages:
        line["stages_flushed"] = measure_stages(b)
    if not args.no_backward:
        line["backward"] = measure_backward(b)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
