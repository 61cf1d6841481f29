"""Benchmark of the Muse Spark Open attention core on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
for each layer of the workload the key norm/RoPE pass (the first rotating
layer's pass also builds the FP32 RoPE table, in the same launch) and the
fused attention kernel (query norm/RoPE prologue, causal GQA flash attention,
output norm x sigmoid gate epilogue).  The default workload is the 32k-token
four-layer mix (three layers with a 8192-key window and RoPE, one full-causal
layer without RoPE; 64 query heads, 8 KV heads, D = 128).  Inputs are resident
in HBM before the timed region.  Prints one JSON line.  Besides the step it
reports the unfused stages of layer 0 (flushed caches), the other workloads'
fused kernel and flushed norm stages, the backward entry points of layer 0,
and the CPU oracle's rate on a sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --summarize-pmc DIR [DIR ...]   # rocprofv3 counter summary (text)
    python bench.py --summarize-trace DIR           # rocprofv3 kernel-trace table
    python bench.py --workload W --traffic-record FETCH_DIR WRITE_DIR   # HBM traffic record
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
DEFAULT_WORKLOAD = "bshd_1x32768_h64kv8_d128_mix"
# the five configurations; the other four get a sub-record each
CONFIGS = ["bshd_1x128_h4kv1_d64", "bshd_2x4096_h32kv8_d128", "bshd_1x16384_h32kv8_d128_w4096",
           "thd_16seg_h40kv8_d128", "bshd_1x32768_h64kv8_d128_mix"]
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
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


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # a 32k-mix step is ~38 ms, so five warmup steps already cover the ~30 ms
    # the clocks need to settle from idle
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(W.WORKLOADS))
    ap.add_argument("--kv-split", type=int, default=0,
                    help="attention KV-split policy (params.kv_split): 0 automatic, 1 never, n >= 2 n parts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true", help="skip the per-stage (unfused) measurements")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurements")
    ap.add_argument("--no-workloads", action="store_true", help="skip the other configurations' sub-records")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (reference kernel for HBM counters)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="print a text summary of rocprofv3 --pmc CSV result directories and exit")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a table of a rocprofv3 --kernel-trace CSV result directory and exit")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the fused kernel's HBM-traffic record of --workload from two rocprofv3 "
                         "--pmc FETCH_SIZE / WRITE_SIZE CSV runs made with --calibrate-copy, and exit")
    return ap.parse_args(argv)


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
    """A workload's layers resident on the GPU, with every buffer the step
    needs (outputs, K-hat, the RoPE table, split workspaces) allocated once."""

    def __init__(self, w: W.Workload, kv_split: int = 0):
        import torch

        import decoder_attention_qk_amd as m
        self.torch, self.m, self.w = torch, m, w
        dev = torch.device("cuda:0")
        self.dev = dev

        def bf(a):
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

        if w.is_thd:
            cu = torch.from_numpy(w.cu_seqlens()).to(dev)
            self.layout = m.Layout.thd(cu, w.max_seqlen, total_tokens=w.tokens)
        else:
            self.layout = m.Layout.bshd(w.batch, w.seqlen)
        self.layers = []
        for li in range(len(w.layers)):
            x = W.make_layer_inputs(w, li)
            p = m.AttnParams(head_dim=w.head_dim, num_heads=w.num_heads,
                             num_key_value_heads=w.num_kv_heads, sliding_window=x["window"],
                             use_rope=x["use_rope"], scaling=float(np.float32(w.head_dim ** -0.5)),
                             qk_eps=EPS, out_eps=EPS, kv_split=kv_split)
            t = dict(params=p, q=bf(x["q"]), k=bf(x["k"]), v=bf(x["v"]), gate=bf(x["gate"]),
                     q_gain=torch.from_numpy(x["q_gain"]).to(dev),
                     k_gain=torch.from_numpy(x["k_gain"]).to(dev), window=x["window"])
            t["k_hat"] = torch.empty_like(t["k"])
            t["out"] = torch.empty_like(t["q"])
            ws = m.muse_attn_fwd_workspace_size(p, self.layout)
            t["ws"] = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None
            self.layers.append(t)
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
                                  t["q_gain"], cos, sin, out=t["out"], workspace=t["ws"])
            if ev is not None:
                ev[3 + 3 * li].record()

    def n_events(self):
        return 1 + 3 * len(self.layers)

    def free(self):
        self.layers.clear()
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def time_steps(b: Bench, steps: int, warmup: int) -> dict:
    """Warmup, then `steps` timed steps bracketed by device synchronisation,
    with events around every launch (a step holds few long launches, so the
    marker packets cost well under 1 %)."""
    torch = b.torch
    for _ in range(warmup):
        b.step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(b.n_events())] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        b.step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nl = len(b.layers)
    attn = np.array([[evs[i][2 + 3 * li].elapsed_time(evs[i][3 + 3 * li]) * 1e-3 for li in range(nl)]
                     for i in range(steps)])
    kpass = np.array([[evs[i][1 + 3 * li].elapsed_time(evs[i][2 + 3 * li]) * 1e-3 for li in range(nl)]
                      for i in range(steps)])
    flop_layers = [layer_flop(b.w, t["window"]) for t in b.layers]
    return dict(step_s=wall / steps, attn_s=attn, kpass_s=kpass, flop_layers=flop_layers)


NOMINAL_CLOCK_MHZ = 2400.0     # the clock the 2.5 PFLOP/s dense bf16 peak is quoted at


def sclk_table_path(torch, dev):
    """The sysfs shader-clock table of the device in use: found by its PCI
    address; else the only such table on the host; else None (several
    tables and no address to tell them apart)."""
    import glob
    try:
        pr = torch.cuda.get_device_properties(dev)
        addr = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
        path = f"/sys/bus/pci/devices/{addr}/pp_dpm_sclk"
        if os.path.exists(path):
            return path
    except (AttributeError, RuntimeError, TypeError, ValueError):
        pass
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    return paths[0] if len(paths) == 1 else None


def current_sclk_mhz(text: str):
    """The current shader clock (MHz) in the text of a pp_dpm_sclk table: the
    level line marked with '*' (e.g. "1: 1844Mhz *"); None if no line is."""
    import re
    for line in text.splitlines():
        if line.rstrip().endswith("*"):
            m = re.search(r"(\d+)\s*Mhz", line, re.IGNORECASE)
            return int(m.group(1)) if m else None
    return None


def clock_under_load(b: Bench, seconds: float = 0.6):
    """Median shader clock (MHz) of the device in use while the step repeats,
    read from the driver's sysfs clock table (the line marked as current in
    pp_dpm_sclk, the value rocm-smi reports) by a thread of this process;
    None where the table is missing or cannot be told apart from other
    devices'.  Runs after the timed steps, so the timed region carries no
    polling."""
    import threading
    path = sclk_table_path(b.torch, b.dev)
    if path is None:
        return None

    def current():
        try:
            with open(path) as f:
                return current_sclk_mhz(f.read())
        except OSError:
            return None

    vals, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            v = current()
            if v:
                vals.append(v)
            stop.wait(0.02)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        b.step()
        b.torch.cuda.synchronize()
    stop.set()
    th.join(timeout=5)
    return float(np.median(vals)) if vals else None


def kernel_record(b: Bench, t: dict) -> dict:
    """The fused attention kernel's roofline record: algorithmic flop per
    launch averaged over the step's launches / the average launch duration."""
    flop = np.array(t["flop_layers"], dtype=np.float64)
    attn = t["attn_s"]
    achieved = float(flop.sum() / attn.mean(axis=0).sum()) / 1e12
    kb = b.layers[0]["k"].numel() * 2
    kp = float(t["kpass_s"].mean())
    return {
        "kernel": f"attn_fwd_kernel<{b.w.head_dim},fused>",
        "achieved": round(achieved, 3), "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "launch_us": round(float(attn.mean()) * 1e6, 2),
        "launch_us_per_layer": [round(float(x) * 1e6, 2) for x in attn.mean(axis=0)],
        "k_norm_rope": {"launch_us": round(kp * 1e6, 2), "GBps": round(2 * kb / kp / 1e9, 1),
                        "frac_hbm": round(2 * kb / kp / 1e9 / PEAK_HBM_GBPS, 4)},
    }


def measure_stages(b: Bench, iters: int = 5, which=("qk_norm_rope", "gqa_attn_fwd", "out_norm_gate",
                                                    "k_norm_rope", "attn_fused_fwd_flushed")) -> dict:
    """Unfused stages of layer 0, each timed alone after reading a 512 MiB
    buffer, which refills the 256 MB Infinity Cache with clean unrelated
    lines, so the HBM-bound kernels are charged HBM traffic (a write-based
    flush would leave dirty lines for the measured kernel to write back)."""
    torch, m, w = b.torch, b.m, b.w
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=b.dev)
    t = b.layers[0]
    p = t["params"]
    cos, sin = (b.cos, b.sin) if p.use_rope else (None, None)
    if p.use_rope:
        m.muse_rope_cos_sin(w.theta, w.head_dim, b.n_pos, b.cos, b.sin)
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
    flop = layer_flop(w, t["window"])
    m.muse_qk_norm_rope(p, b.layout, t["q"], t["k"], t["q_gain"], t["k_gain"], cos, sin, q_out=q_hat,
                        k_out=k_hat)
    m.muse_gqa_attn_fwd(p, b.layout, q_hat, k_hat, t["v"], o=o, workspace=t["ws"])
    res = {}
    if "qk_norm_rope" in which:
        s = timed(lambda: m.muse_qk_norm_rope(p, b.layout, t["q"], t["k"], t["q_gain"], t["k_gain"], cos, sin,
                                              q_out=q_hat, k_out=k_hat))
        res["qk_norm_rope"] = dict(us=s * 1e6, GBps=2 * (qb + kb) / s / 1e9)
    if "gqa_attn_fwd" in which:
        s = timed(lambda: m.muse_gqa_attn_fwd(p, b.layout, q_hat, k_hat, t["v"], o=o, workspace=t["ws"]))
        res["gqa_attn_fwd"] = dict(us=s * 1e6, TFLOPs=flop / s / 1e12)
    if "out_norm_gate" in which:
        s = timed(lambda: m.muse_out_norm_gate(p, b.layout, o, t["gate"], out=out))
        res["out_norm_gate"] = dict(us=s * 1e6, GBps=3 * qb / s / 1e9)
    if "k_norm_rope" in which:
        s = timed(lambda: m.muse_qk_norm_rope(p, b.layout, None, t["k"], None, t["k_gain"], cos, sin,
                                              k_out=k_hat))
        res["k_norm_rope"] = dict(us=s * 1e6, GBps=2 * kb / s / 1e9)
    if "attn_fused_fwd_flushed" in which:
        s = timed(lambda: m.muse_attn_fused_fwd(p, b.layout, t["q"], k_hat, t["v"], t["gate"], t["q_gain"], cos,
                                                sin, out=out, workspace=t["ws"]))
        res["attn_fused_fwd_flushed"] = dict(us=s * 1e6, TFLOPs=flop / s / 1e12)
    for v in res.values():
        if "GBps" in v:
            v["frac_hbm"] = v["GBps"] / PEAK_HBM_GBPS
        if "TFLOPs" in v:
            v["frac_mfma"] = v["TFLOPs"] / PEAK_BF16_TFLOPS
        for key in list(v):
            v[key] = round(v[key], 4)
    del flush
    return res


def measure_backward(b: Bench, warmup: int = 5, iters: int = 20) -> dict:
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
    if p.use_rope:
        m.muse_rope_cos_sin(w.theta, w.head_dim, b.n_pos, b.cos, b.sin)
    q_hat, k_hat, _, _ = m.muse_qk_norm_rope(p, lay, t["q"], t["k"], t["q_gain"], t["k_gain"], cos, sin)
    o, lse = m.muse_gqa_attn_fwd(p, lay, q_hat, k_hat, t["v"], want_lse=True, workspace=t["ws"])
    g = torch.Generator(device=b.dev)
    g.manual_seed(7)
    dout = torch.randn(t["q"].shape, generator=g, device=b.dev).to(torch.bfloat16)

    def ws(n):
        return torch.empty(max(1, n), dtype=torch.uint8, device=b.dev)
    ws_attn = ws(m.muse_gqa_attn_bwd_workspace_size(p, lay))
    size = ctypes.c_size_t(0)
    pc, lc = p.to_c(), lay.to_c()
    m.library().muse_qk_norm_rope_bwd_workspace_size(ctypes.byref(pc), ctypes.byref(lc), ctypes.byref(size))
    ws_qk = ws(size.value)
    m.library().muse_attn_core_bwd_workspace_size(ctypes.byref(pc), ctypes.byref(lc), ctypes.byref(size))
    ws_core = ws(size.value)
    d_o, dgate, delta = m.muse_out_norm_gate_bwd(p, lay, o, t["gate"], dout)
    dq_hat, dk_hat, dv = m.muse_gqa_attn_bwd(p, lay, q_hat, k_hat, t["v"], d_o, lse, delta, workspace=ws_attn)
    dq, dk, dqg, dkg = m.muse_qk_norm_rope_bwd(p, lay, t["q"], t["k"], t["q_gain"], t["k_gain"], cos, sin,
                                               dq_hat, dk_hat, workspace=ws_qk)
    res_core = m.muse_attn_core_bwd(p, lay, t["q"], t["k"], t["v"], t["gate"], dout, t["q_gain"], t["k_gain"],
                                    cos, sin, o=o, lse=lse, workspace=ws_core)
    calls = [
        lambda: m.muse_out_norm_gate_bwd(p, lay, o, t["gate"], dout, d_o=d_o, dgate=dgate, delta=delta),
        lambda: m.muse_gqa_attn_bwd(p, lay, q_hat, k_hat, t["v"], d_o, lse, delta, dq_hat=dq_hat,
                                    dk_hat=dk_hat, dv=dv, workspace=ws_attn),
        lambda: m.muse_qk_norm_rope_bwd(p, lay, t["q"], t["k"], t["q_gain"], t["k_gain"], cos, sin, dq_hat,
                                        dk_hat, dq=dq, dk=dk, dq_gain=dqg, dk_gain=dkg, workspace=ws_qk),
        lambda: m.muse_attn_core_bwd(p, lay, t["q"], t["k"], t["v"], t["gate"], dout, t["q_gain"],
                                     t["k_gain"], cos, sin, o=o, lse=lse, dq=res_core[0], dk=res_core[1],
                                     dv=res_core[2], dgate=res_core[3], dq_gain=res_core[4],
                                     dk_gain=res_core[5], workspace=ws_core),
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
        "layer": 0,
        "out_norm_gate_bwd": {"us": round(us[0], 2), "GBps": round(5 * qb / us[0] / 1e3, 1),
                              "frac_hbm": round(5 * qb / us[0] / 1e3 / PEAK_HBM_GBPS, 4)},
        "gqa_attn_bwd": {"us": round(us[1], 2), "TFLOPs": round(flop / us[1] / 1e6, 2),
                         "frac_mfma": round(flop / us[1] / 1e6 / PEAK_BF16_TFLOPS, 4),
                         "flop_algorithmic": int(flop)},
        "qk_norm_rope_bwd": {"us": round(us[2], 2), "GBps": round(3 * (qb + kb) / us[2] / 1e3, 1),
                             "frac_hbm": round(3 * (qb + kb) / us[2] / 1e3 / PEAK_HBM_GBPS, 4)},
        "attn_core_bwd": {"us": round(us[3], 2), "TFLOPs": round(flop / us[3] / 1e6, 2)},
    }


def measure_workload(name: str, kv_split: int, warm_s: float = 0.1, timed_s: float = 0.2) -> dict:
    """Sub-record of another configuration: its step, the fused kernel's
    roofline fraction and the flushed Q/K norm+RoPE and output norm/gate stages.
    Warmup and timed steps are counted to cover about warm_s and timed_s of
    work (at least 5 and 10 steps), so short steps still run at settled clocks."""
    w = W.WORKLOADS[name]
    b = Bench(w, kv_split)
    b.step()
    b.torch.cuda.synchronize()
    t0 = time.perf_counter()
    b.step()
    b.torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-6)
    t = time_steps(b, max(10, int(timed_s / one)), max(5, int(warm_s / one)))
    rec = kernel_record(b, t)
    flop_step = sum(t["flop_layers"])
    st = measure_stages(b, which=("qk_norm_rope", "out_norm_gate"))
    out = {"steps": len(t["attn_s"]), "step_ms": round(t["step_s"] * 1e3, 4),
           "TFLOPs_step": round(flop_step / t["step_s"] / 1e12, 3),
           "fused_kernel": rec, "qk_norm_rope_flushed": st["qk_norm_rope"],
           "out_norm_gate_flushed": st["out_norm_gate"]}
    b.free()
    return out


def cpu_baseline(w: W.Workload, budget_s: float = 20.0) -> dict:
    """The FP64 oracle, as it stands, on a sample of the same workload: per
    layer its key-side work (norm + RoPE of every key) once, and the full path
    (query norm/RoPE, attention, norm-gate) of sampled (token, head) rows; the
    step time is extrapolated from the measured key-side time and the rows'
    time per visible (query, key) pair, over every row of every layer."""
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(0)
    segs = O.Segments.thd(w.cu_seqlens()) if w.is_thd else O.Segments.bshd(w.batch, w.seqlen)
    pos = segs.local_positions()
    kw = dict(theta=w.theta, eps=EPS, out_eps=EPS, scaling=float(np.float32(w.head_dim ** -0.5)))
    # layers with the same (window, rope) share one measurement
    kinds = {}
    for li, (win, rope) in enumerate(w.layers):
        kinds.setdefault((win, rope), li)
    per_layer_budget = budget_s / len(kinds)
    total_s = 0.0
    sample_rows = 0
    sample_s = 0.0
    meas = {}
    for (win, rope), li in kinds.items():
        x = W.make_layer_inputs(w, li)
        qg, kg = x["q_gain"].astype(np.float64), x["k_gain"].astype(np.float64)
        k64, v64 = O.bf16_bits_to_f64(x["k"]), O.bf16_bits_to_f64(x["v"])

        def run(rows):
            tok = np.array([r[0] for r in rows])
            hd = np.array([r[1] for r in rows])
            t0 = time.perf_counter()
            O.attn_core_rows(O.bf16_bits_to_f64(x["q"][tok, hd]), k64, v64, O.bf16_bits_to_f64(x["gate"][tok, hd]),
                             segs, rows, num_heads=w.num_heads, window=win, use_rope=rope, q_gain=qg,
                             k_gain=kg, **kw)
            return time.perf_counter() - t0

        def pairs_of(rows):
            return sum(min(int(pos[t]) + 1, win) if win > 0 else int(pos[t]) + 1 for t, _ in rows)

        def draw(n):
            return [(int(rng.integers(w.tokens)), int(rng.integers(w.num_heads))) for _ in range(n)]
        one = draw(1)
        t1 = run(one)
        n = 16
        rows = draw(n)
        tn = run(rows)
        # grow the sample until it takes about the layer's share of the budget
        while tn < 0.5 * per_layer_budget and n < 65536:
            n = min(65536, int(n * max(2.0, 0.6 * per_layer_budget / max(tn, 1e-3))))
            rows = draw(n)
            tn = run(rows)
        p1, pn = pairs_of(one), pairs_of(rows)
        per_pair = max(tn - t1, 1e-9) / max(pn - p1, 1)
        key_side = max(t1 - p1 * per_pair, 0.0)
        meas[(win, rope)] = (key_side, per_pair)
        sample_rows += n + 1
        sample_s += t1 + tn
    flop_step = 0
    for win, rope in w.layers:
        key_side, per_pair = meas[(win, rope)]
        pairs = w.num_heads * sum(visible_pairs(L, win) for L in seq_lengths(w))
        total_s += key_side + per_pair * pairs
        flop_step += 4 * w.head_dim * pairs
    return {"value": round(flop_step / total_s / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "extrapolated": True,
            "sample": f"{sample_rows} (token, head) rows over {len(kinds)} layer kinds in {sample_s:.1f} s of "
                      f"oracle time (full path per row: query norm/RoPE, attention, norm-gate; plus every key's "
                      f"norm/RoPE per layer); the step's {total_s:.0f} s is extrapolated from the key-side time "
                      f"and the time per visible (query, key) pair; BLAS threads as numpy sets them on "
                      f"{cores} cores, elementwise numpy single-threaded"}


def _csv_rows(d: str, suffix: str) -> list[dict]:
    """Rows of every rocprofv3 CSV file under d whose name ends in suffix."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _short_kernel(name: str) -> str:
    return name.replace("muse::(anonymous namespace)::", "").replace("(anonymous namespace)::", "") \
        .replace("muse::", "").split("(")[0].replace("void ", "").strip()


def _counter_table(d: str) -> dict:
    """{dispatch id: (kernel, {counter: value summed over instances})} of a
    rocprofv3 --pmc CSV directory."""
    import collections
    per = collections.OrderedDict()
    for r in _csv_rows(d, "counter_collection.csv"):
        did = int(r["Dispatch_Id"])
        name, vals = per.setdefault(did, (_short_kernel(r["Kernel_Name"]), collections.defaultdict(float)))
        vals[r["Counter_Name"]] += float(r["Counter_Value"])
    return per


def summarize_trace(d: str) -> str:
    """Markdown table of a rocprofv3 --kernel-trace CSV directory: per kernel
    and grid, the number of dispatches and their mean, min and max duration."""
    import collections
    groups = collections.OrderedDict()
    for r in _csv_rows(d, "kernel_trace.csv"):
        grid = int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0)
        key = (_short_kernel(r["Kernel_Name"]), grid)
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["| kernel | grid (threads) | calls | mean us | min us | max us |", "|---|---|---|---|---|---|"]
    for (name, grid), us in groups.items():
        lines.append(f"| {name} | {grid} | {len(us)} | {np.mean(us):.2f} | {min(us):.2f} | {max(us):.2f} |")
    return "\n".join(lines)


def summarize_pmc(dirs: list[str]) -> str:
    """Text summary of rocprofv3 --pmc CSV directories: per kernel, the mean
    of each counter per dispatch and the ratios the attention kernel's
    analysis uses."""
    import collections
    lines = []
    for d in dirs:
        per = _counter_table(d)
        agg = collections.OrderedDict()
        for name, vals in per.values():
            n, tot = agg.setdefault(name, [0, collections.defaultdict(float)])
            agg[name][0] += 1
            for k, v in vals.items():
                tot[k] += v
        lines.append(f"## {os.path.basename(os.path.normpath(d))}")
        # HBM counters calibrated on the 256 MiB copy of --calibrate-copy, when present
        scale = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            copies = [v[counter] for name, v in per.values() if name.startswith("__amd_rocclr_copyBuffer") and counter in v]
            if copies and max(copies) > 0:
                scale[counter] = 256 * 1024 * 1024 / (max(copies) * 1024.0)
        for name, (n, tot) in agg.items():
            c = {k: v / n for k, v in tot.items()}
            lines.append(f"- `{name}`: {n} dispatches; per dispatch: "
                         + ", ".join(f"{k} {v:.6g}" for k, v in sorted(c.items())))
            mf = c.get("SQ_INSTS_MFMA", 0.0)
            r = []
            if mf:
                if "SQ_INSTS_VALU" in c:
                    r.append(f"non-MFMA VALU per MFMA {(c['SQ_INSTS_VALU'] - mf) / mf:.3f}")
                for k in ("SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
                    if k in c:
                        r.append(f"{k} per MFMA {c[k] / mf:.3f}")
            if c.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in c:
                r.append(f"VALU co-issued with MFMA in {c['SQ_VALU_MFMA_COEXEC_CYCLES'] / c['SQ_VALU_MFMA_BUSY_CYCLES']:.3f}"
                         " of MFMA-busy cycles")
            for counter, sc in scale.items():
                if counter in c:
                    r.append(f"{counter} x {sc:.4f} = {c[counter] * 1024.0 * sc / 1e9:.4f} GB per dispatch")
            if c.get("SQ_VALU_MFMA_BUSY_CYCLES") and c.get("SQ_BUSY_CU_CYCLES"):
                r.append(f"MFMA busy per SIMD-cycle of a busy CU (SQ_VALU_MFMA_BUSY_CYCLES / (4 SQ_BUSY_CU_CYCLES)) "
                         f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * c['SQ_BUSY_CU_CYCLES']):.3f}")
            if c.get("SQ_WAVE_CYCLES") and c.get("SQ_BUSY_CU_CYCLES"):
                r.append(f"waves resident per busy CU (4 SQ_WAVE_CYCLES / SQ_BUSY_CU_CYCLES; wave cycles count "
                         f"in units of 4) {4 * c['SQ_WAVE_CYCLES'] / c['SQ_BUSY_CU_CYCLES']:.2f}")
            if r:
                lines.append("  - " + "; ".join(r))
    return "\n".join(lines)


def traffic_record(workload: str, fetch_dir: str, write_dir: str) -> dict:
    """HBM bytes per launch of the fused attention kernel from two rocprofv3
    --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by
    what the same counter reads for the 256 MiB device copy of
    --calibrate-copy (the largest copy dispatch of the run)."""
    copy_bytes = 256 * 1024 * 1024
    w = W.WORKLOADS[workload]
    out = {"workload": workload, "kernel": f"attn_fwd_kernel<{w.head_dim}, true, false>",
           "kernel_source_digest": kernel_source_digest()}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _counter_table(d)
        copies = [v[counter] for name, v in per.values() if name.startswith("__amd_rocclr_copyBuffer") and counter in v]
        fused = [v[counter] for name, v in per.values() if name.startswith("attn_fwd_kernel") and "true" in name
                 and counter in v]
        if not copies or not fused:
            raise SystemExit(f"{d}: no copy or fused-attention dispatch with {counter}")
        scale = copy_bytes / (max(copies) * 1024.0)
        key = "fetch" if counter == "FETCH_SIZE" else "write"
        out[f"{key}_bytes_per_launch"] = int(round(np.mean(fused) * 1024.0 * scale))
        out[f"{key}_scale"] = round(scale, 4)
    qb = w.tokens * w.num_heads * w.head_dim * 2
    kb = w.tokens * w.num_kv_heads * w.head_dim * 2
    out["algorithmic_read_bytes"] = 2 * qb + 2 * kb
    out["algorithmic_write_bytes"] = qb
    # the attention backward's two kernels, when the runs included it: each
    # reads q-hat, dO, k-hat, v, LSE and delta once; dQ writes dq-hat, dK/dV
    # writes dk-hat and dv
    rows = w.tokens * w.num_heads * 4
    bwd = {}
    for kname, wbytes in (("attn_bwd_dq_kernel", qb), ("attn_bwd_dkdv", 2 * kb)):
        rec = {"algorithmic_read_bytes": 2 * qb + 2 * kb + 2 * rows, "algorithmic_write_bytes": wbytes}
        for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
            per = _counter_table(d)
            vals = [v[counter] for name, v in per.values() if name.startswith(kname) and counter in v]
            if not vals:
                break
            key = "fetch" if counter == "FETCH_SIZE" else "write"
            rec[f"{key}_bytes_per_launch"] = int(round(np.mean(vals) * 1024.0 * out[f"{key}_scale"]))
        else:
            rec["fetched_over_algorithmic"] = round(rec["fetch_bytes_per_launch"] / rec["algorithmic_read_bytes"], 3)
            bwd[kname] = rec
    if bwd:
        out["backward"] = bwd
    return out


def main(argv=None):
    args = parse(argv)
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.traffic_record:
        print(json.dumps(traffic_record(args.workload, *args.traffic_record), indent=1))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): the library has no "
              "multi-GPU path; each GPU would run it on its own share of the KV heads", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    w = W.WORKLOADS[args.workload]
    b = Bench(w, args.kv_split)
    if args.calibrate_copy:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=b.dev)   # 256 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    t = time_steps(b, args.steps, args.warmup)
    rec = kernel_record(b, t)
    flop_step = sum(t["flop_layers"])
    kb = b.layers[0]["k"].numel() * 2
    qb = b.layers[0]["q"].numel() * 2
    line = {
        "metric": METRIC,
        "value": round(flop_step / t["step_s"] / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["step_s"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "tokens": w.tokens, "batch": w.batch if not w.is_thd else 1,
            "seq_len": w.max_seqlen, "segments": len(seq_lengths(w)), "num_heads": w.num_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "layers": [{"sliding_window": t_["window"], "use_rope": bool(t_["params"].use_rope)}
                       for t_ in b.layers],
            "flop_per_step_causal": flop_step,
            "share_of": W.SHARE_OF.get(w.name),
            "kv_split_policy": args.kv_split,
        },
        "roofline": {
            "bound": "mfma", "kernel": rec["kernel"],
            "achieved": rec["achieved"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": rec["frac"], "traffic": measured_traffic(w.name, len(b.layers)),
            "launch_us": rec["launch_us"], "launch_us_per_layer": rec["launch_us_per_layer"],
            "kernel_source_digest": kernel_source_digest(),
        },
        "k_norm_rope": rec["k_norm_rope"],
        "fused_bytes_per_layer": 3 * qb + 2 * kb,
    }
    # for information: the same fraction against the peak scaled to the shader
    # clock measured under the step's load
    clk = clock_under_load(b)
    line["roofline"]["clock_mhz_under_load"] = clk
    line["roofline"]["frac_at_clock"] = (
        round(rec["achieved"] / (PEAK_BF16_TFLOPS * clk / NOMINAL_CLOCK_MHZ), 4) if clk else None)
    if not args.no_stages:
        line["stages_flushed"] = measure_stages(b)
    if not args.no_backward:
        line["backward"] = measure_backward(b)
    b.free()
    del b
    if not args.no_workloads and w.name in CONFIGS:
        line["workloads"] = {}
        for name in CONFIGS:
            if name != w.name:
                line["workloads"][name] = measure_workload(name, args.kv_split)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
