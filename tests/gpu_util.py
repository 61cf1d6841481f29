"""Helpers for GPU parity tests: moving seeded inputs to the device, building
oracle inputs from the same bits, and the tolerance checks.

Tolerances (the 2e-2 / 1e-5 bar, made concrete):
* bf16 outputs: for every (token, head) row, max_d |g - r| <= 2e-2 * max_d |r|
  (the row's max relative error).  The method itself puts elementwise errors
  near 2e-2 of an element's own size in rare tails: P is rounded to bf16 for
  the PV product (as the pages' SDPA/TE path does), and the attention output
  and the gated output are two bf16 boundaries that may each legitimately
  differ by one ulp (2^-7 relative at worst).  The elementwise error scaled by
  max(|r|, rms_row) is still computed and reported;
* FP32 intermediates (rstd, lse): |g - r| <= 1e-5 * max(|r|, floor), r the
  oracle evaluated on the GPU's own bf16 inputs to that stage (floor 1 for
  lse, which is a log and can sit near 0; 0 for rstd).
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

import decoder_attention_qk_amd as m
import oracle as O
import workloads as W

EPS = 1e-6
BF16_TOL = 2e-2
FP32_TOL = 1e-5


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits_f64(bits: np.ndarray) -> np.ndarray:
    return O.bf16_bits_to_f64(bits)


def check_bf16(got: np.ndarray, ref: np.ndarray, tol: float = BF16_TOL, what: str = "") -> dict:
    if got.size == 0:
        return dict(max_err=0.0, elem_err=0.0, exact=1.0)
    diff = np.abs(got - ref)
    row_max = np.abs(ref).max(axis=-1, keepdims=True)
    row_err = diff.max(axis=-1, keepdims=True) / np.where(row_max == 0, 1.0, row_max)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    elem = diff / np.where(np.maximum(np.abs(ref), rms) == 0, 1.0, np.maximum(np.abs(ref), rms))
    stats = dict(max_err=float(row_err.max()), elem_err=float(elem.max()), exact=float(np.mean(got == ref)))
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    assert stats["max_err"] <= tol, f"{what}: row max relative error {stats['max_err']:.4g} > {tol} ({stats})"
    return stats


def check_fp32(got: np.ndarray, ref: np.ndarray, tol: float = FP32_TOL, floor: float = 0.0,
               what: str = "") -> float:
    err = np.abs(got - ref) / np.maximum(np.abs(ref), floor)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max rel error {worst:.3g} > {tol}"
    return worst


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


def sample_rows(segs: O.Segments, num_heads: int, window: int, n_random: int, seed: int = 0):
    """Deterministic (token, head) sample: every segment's first and last rows,
    rows around the window edge after each start, and random rows over all heads."""
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
    total = segs.total
    for _ in range(n_random):
        rows.add((int(rng.integers(total)), int(rng.integers(num_heads))))
    return sorted(rows)
