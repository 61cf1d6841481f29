"""Helpers for GPU parity tests: moving seeded inputs to the device, building
oracle inputs from the same bits, and the tolerance checks.

Tolerances (the 2e-2 / 1e-5 bar, made concrete):
* bf16 outputs, two bars, both asserted:
  - the row bar: for every (token, head) row, max_d |g - r| <= 2e-2 * max_d |r|;
  - the elementwise bar: |g - r| <= ELEM_TOL * max(|r|, rms_row(r)) for every
    element.  ELEM_TOL = 3e-2 is the sum of what the method itself allows:
    the final bf16 boundary may round the other way (one ulp, <= 2^-7 of the
    element), so may the attention output's bf16 boundary before the output
    norm (another 2^-7 of the element after the norm and gate), and the
    probabilities are rounded to bf16 for the PV product as the pages'
    SDPA/TE path does (independent round-to-nearest errors of at most half an
    ulp; their sum over keys has a standard deviation of at most
    2^-7 / sqrt(12) of the row's RMS, and six of those are allowed):
    2 * 2^-7 + 6 * 2^-7 / sqrt(12) = 0.0286 < 3e-2.
  Gradients (the backward tests) assert the row bar and record the
  elementwise figure (elem_tol=None): the pages state no gradient tolerance,
  and cancellation makes an elementwise bound on them data-dependent;
* FP32 intermediates (rstd, lse): |g - r| <= 1e-5 * max(|r|, floor), r the
  oracle evaluated on the GPU's own bf16 inputs to that stage (floor 1 for
  lse, which is a log and can sit near 0; 0 for rstd).

Every check's row and elementwise figures are recorded in RESULTS; the test
session prints the worst of them per test at its end.
"""

from __future__ import annotations

import math
import os

import dataclasses

import numpy as np
import torch

import decoder_attention_qk_amd as m
import oracle as O
import workloads as W

EPS = 1e-6
BF16_TOL = 2e-2
ELEM_TOL = 3e-2
assert 2 * 2.0 ** -7 + 6 * 2.0 ** -7 / math.sqrt(12) < ELEM_TOL
FP32_TOL = 1e-5
RESULTS: list = []   # one dict per bf16 check (test, what, max_err, elem_err, exact, elements)


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits_f64(bits: np.ndarray) -> np.ndarray:
    return O.bf16_bits_to_f64(bits)


def check_bf16(got: np.ndarray, ref: np.ndarray, tol: float = BF16_TOL, what: str = "",
               elem_tol: float | None = ELEM_TOL) -> dict:
    """Asserts the row bar (tol) and, unless elem_tol is None, the elementwise
    bar; returns and records both figures."""
    if got.size == 0:
        return dict(max_err=0.0, elem_err=0.0, exact=1.0)
    diff = np.abs(got - ref)
    row_max = np.abs(ref).max(axis=-1, keepdims=True)
    row_err = diff.max(axis=-1, keepdims=True) / np.where(row_max == 0, 1.0, row_max)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    scale = np.maximum(np.abs(ref), rms)
    elem = np.where(scale == 0, diff, diff / np.where(scale == 0, 1.0, scale))
    stats = dict(max_err=float(row_err.max()), elem_err=float(elem.max()), exact=float(np.mean(got == ref)))
    RESULTS.append(dict(test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], what=what,
                        elements=int(got.size), **stats))
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    assert stats["max_err"] <= tol, f"{what}: row max relative error {stats['max_err']:.4g} > {tol} ({stats})"
    if elem_tol is not None:
        assert stats["elem_err"] <= elem_tol, \
            f"{what}: elementwise error {stats['elem_err']:.4g} > {elem_tol} of max(|r|, rms_row) ({stats})"
    return stats


def check_fp32(got: np.ndarray, ref: np.ndarray, tol: float = FP32_TOL, floor: float = 0.0,
               what: str = "") -> float:
    err = np.abs(got - ref) / np.maximum(np.abs(ref), floor)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max rel error {worst:.3g} > {tol}"
    return worst


def check_scaled(got, ref, scale, what, tol=BF16_TOL):
    """Row max error within tol of the row max of a magnitude bound: the
    backward's sums cancel (dS sums to zero over each softmax row, the norm
    backward removes the component along x), so a result can be far smaller
    than the terms it is summed from, and its rounding error scales with the
    terms.  ``scale`` is the same computation carried out on magnitudes."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    err = np.abs(got - ref).max(axis=-1)
    bound = tol * np.abs(scale).max(axis=-1)
    worst = float((err / np.maximum(bound, 1e-30)).max())
    assert np.all(err <= bound), f"{what}: worst {worst:.3g} of the bound"
    return worst


def core_bwd_magnitudes(case, dout_f64, ref, kw):
    """Magnitude bounds of dq, dk, dv, dgate and the gain gradients of the
    whole backward, stage by stage on the oracle's own forward values."""
    fw = O.attn_core(bits_f64(case.x["q"]), bits_f64(case.x["k"]), bits_f64(case.x["v"]),
                     bits_f64(case.x["gate"]), case.segs, **kw)
    o, r_o = fw["o"], fw["o_rstd"][..., None]
    sig = 1.0 / (1.0 + np.exp(-bits_f64(case.x["gate"])))
    dy_a = np.abs(dout_f64) * sig
    do_a = r_o * dy_a + r_o ** 3 * np.abs(o) * np.mean(dy_a * np.abs(o), axis=-1, keepdims=True)
    y = o * r_o
    dgate_a = np.abs(dout_f64 * y * sig * (1.0 - sig))
    _, _, _, dqh_a, dkh_a, dv_a = O.attention_bwd(fw["q_hat"], fw["k_hat"], bits_f64(case.x["v"]), ref["d_o"],
                                                  case.segs, window=kw["window"], scaling=kw["scaling"], o=o,
                                                  mags=True, d_o_abs=do_a, causal=kw.get("causal", True),
                                                  key_valid=kw.get("key_valid"))

    def back(g_a, x_bits, gain, qs):
        if kw["use_rope"]:
            pair = g_a[..., 0::2] + g_a[..., 1::2]
            g_a = np.repeat(pair, 2, axis=-1)
        g_a = g_a * abs(qs)
        x = bits_f64(x_bits)
        xn, r = O.rms_normalize(x, EPS)
        r = r[..., None]
        w = np.abs(1.0 + gain) if gain is not None else 1.0
        u = g_a * w
        dx_a = r * u + r ** 3 * np.abs(x) * np.mean(u * np.abs(x), axis=-1, keepdims=True)
        gain_a = np.sum((g_a * np.abs(xn)).reshape(-1, x.shape[-1]), axis=0)
        return dx_a, gain_a

    dq_a, dqg_a = back(dqh_a, case.x["q"], kw["q_gain"], kw["query_scale"])
    dk_a, dkg_a = back(dkh_a, case.x["k"], kw["k_gain"], 1.0)
    return dict(dq=dq_a, dk=dk_a, dv=dv_a, dgate=dgate_a, dq_gain=dqg_a, dk_gain=dkg_a)


@dataclasses.dataclass
class Case:
    """A workload layer on the GPU plus the matching oracle inputs."""

    w: W.Workload
    layer: int
    x: dict
    params: m.AttnParams
    layout: m.Layout
    segs: O.Segments
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    gate: torch.Tensor
    q_gain: torch.Tensor
    k_gain: torch.Tensor
    cos: torch.Tensor | None
    sin: torch.Tensor | None
    n_pos: int

    @property
    def scaling(self) -> float:
        return float(np.float32(self.w.head_dim ** -0.5))

    def oracle_kw(self) -> dict:
        return dict(theta=self.w.theta, eps=self.params.qk_eps, out_eps=self.params.out_eps,
                    scaling=self.scaling, window=self.x["window"], use_rope=self.x["use_rope"],
                    q_gain=self.x["q_gain"].astype(np.float64),
                    k_gain=self.x["k_gain"].astype(np.float64),
                    query_scale=self.params.query_scale, gain_center=self.params.gain_center,
                    upcast_rope=bool(self.params.upcast_rope), causal=not self.params.bidirectional)


def make_case(w: W.Workload, layer: int = 0, *, query_scale: float = 1.0, upcast_rope: bool = True,
              bidirectional: bool = False, device="cuda") -> Case:
    x = W.make_layer_inputs(w, layer)
    params = m.AttnParams(head_dim=w.head_dim, num_heads=w.num_heads,
                          num_key_value_heads=w.num_kv_heads, sliding_window=x["window"],
                          use_rope=x["use_rope"], upcast_rope=upcast_rope, bidirectional=bidirectional,
                          scaling=float(np.float32(w.head_dim ** -0.5)),
                          query_scale=query_scale, qk_eps=EPS, out_eps=EPS)
    if w.is_thd:
        cu = torch.from_numpy(x["cu_seqlens"]).to(device)
        layout = m.Layout.thd(cu, w.max_seqlen, total_tokens=w.tokens)
        segs = O.Segments.thd(x["cu_seqlens"])
    else:
        layout = m.Layout.bshd(w.batch, w.seqlen)
        segs = O.Segments.bshd(w.batch, w.seqlen)
    n_pos = max(1, w.max_seqlen)
    cos = sin = None
    if x["use_rope"]:
        cos, sin = m.muse_rope_cos_sin(w.theta, w.head_dim, n_pos, device=device)
    return Case(w, layer, x, params, layout, segs, dev_bf16(x["q"], device), dev_bf16(x["k"], device),
                dev_bf16(x["v"], device), dev_bf16(x["gate"], device),
                torch.from_numpy(x["q_gain"]).to(device), torch.from_numpy(x["k_gain"]).to(device),
                cos, sin, n_pos)


def sample_rows(segs: O.Segments, num_heads: int, window: int, n_random: int, seed: int = 0,
                num_kv_heads: int | None = None):
    """Deterministic (token, head) sample: every segment's first and last rows,
    rows around the window edge after each start, and random rows over all
    heads.  With num_kv_heads, also one row of every attention work item: the
    forward kernel gives a workgroup 128 (token, head) columns of one KV
    group, G = num_heads / num_kv_heads heads by 128 // G tokens, so every
    (segment, block of 128 // G tokens, KV head) gets a random token of the
    block and a random head of the group."""
    rng = np.random.default_rng(seed)
    rows = set()
    for s0, length in zip(segs.starts, segs.lengths):
        if length == 0:
            continue
        picks = {0, length - 1, min(1, length - 1)}
        if window and window > 0:
            for i in range(window - 2, window + 2):
                if 0 <= i < length:
                    picks.add(i)
        for i in picks:
            rows.add((s0 + i, int(rng.integers(num_heads))))
        if num_kv_heads:
            g = num_heads // num_kv_heads
            tpb = max(1, 128 // g)
            for b0 in range(0, length, tpb):
                toks = rng.integers(b0, min(b0 + tpb, length), num_kv_heads)
                heads = np.arange(num_kv_heads) * g + rng.integers(0, g, num_kv_heads)
                rows.update((s0 + int(t), int(h)) for t, h in zip(toks, heads))
    total = segs.total
    for _ in range(n_random):
        rows.add((int(rng.integers(total)), int(rng.integers(num_heads))))
    return sorted(rows)
