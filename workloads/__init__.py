"""Seeded synthetic workloads for the Muse Spark Open attention core.

This module only draws inputs: shapes, seeds and random tensors.  It holds none
of the method's arithmetic, and both the GPU tests/bench and the CPU oracle
take their inputs from it.

Every tensor has its own numpy PCG64 stream keyed by (seed, config, layer,
tensor name).  Values are drawn as float32 ``standard_normal * std`` and
converted to bfloat16 with torch's round-to-nearest-even cast; tensors are
returned as uint16 bit patterns (bf16) or float32 (gains, already rounded to
bf16-representable values) and int32 (``cu_seqlens``).
"""

from __future__ import annotations

import dataclasses
import zlib

import numpy as np

__all__ = ["Workload", "WORKLOADS", "thd_lengths", "draw_bf16", "draw_gain", "make_layer_inputs",
           "small_workload"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-core workload: geometry plus the per-layer (window, use_rope) mix."""

    name: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    theta: float
    batch: int = 1
    seqlen: int = 0                        # BSHD sequence length (0 for packed THD)
    segment_lengths: tuple = ()            # packed THD segment lengths (empty for BSHD)
    layers: tuple = ((0, True),)           # (sliding_window, use_rope) per layer, 0 = no window
    gate_std: float = 1.0
    gain_std: float = 0.05
    seed: int = 0

    @property
    def is_thd(self) -> bool:
        return len(self.segment_lengths) > 0

    @property
    def tokens(self) -> int:
        return int(sum(self.segment_lengths)) if self.is_thd else self.batch * self.seqlen

    @property
    def max_seqlen(self) -> int:
        return int(max(self.segment_lengths)) if self.is_thd else self.seqlen

    def cu_seqlens(self) -> np.ndarray:
        """int32 [segments + 1] cumulative boundaries (BSHD: one per batch row)."""
        lens = list(self.segment_lengths) if self.is_thd else [self.seqlen] * self.batch
        return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def thd_lengths(seed: int = 0, count: int = 16, low: int = 256, high: int = 8192) -> tuple:
    """Packed segment lengths drawn uniformly from the inclusive range [low, high]."""
    return tuple(int(x) for x in np.random.default_rng(seed).integers(low, high + 1, count))


WORKLOADS = {
    "bshd_1x128_h4kv1_d64": Workload(
        "bshd_1x128_h4kv1_d64", num_heads=4, num_kv_heads=1, head_dim=64, theta=1.0e4,
        batch=1, seqlen=128),
    "bshd_2x4096_h32kv8_d128": Workload(
        "bshd_2x4096_h32kv8_d128", num_heads=32, num_kv_heads=8, head_dim=128, theta=5.0e5,
        batch=2, seqlen=4096),
    "bshd_1x16384_h32kv8_d128_w4096": Workload(
        "bshd_1x16384_h32kv8_d128_w4096", num_heads=32, num_kv_heads=8, head_dim=128,
        theta=5.0e5, batch=1, seqlen=16384, layers=((4096, True),)),
    "thd_16seg_h40kv8_d128": Workload(
        "thd_16seg_h40kv8_d128", num_heads=40, num_kv_heads=8, head_dim=128, theta=5.0e5,
        segment_lengths=thd_lengths(0)),
    "bshd_1x32768_h64kv8_d128_mix": Workload(
        "bshd_1x32768_h64kv8_d128_mix", num_heads=64, num_kv_heads=8, head_dim=128,
        theta=5.0e5, batch=1, seqlen=32768,
        layers=((8192, True), (8192, True), (8192, True), (0, False)), gate_std=4.0),
}

# One GPU's share of the four large workloads when their KV heads are split over
# eight GPUs (one KV head and its query heads per GPU; the heads of a KV group
# need nothing from other groups): the same sequences at 1/8 of the heads.
for _full, _share, _hq in (("bshd_2x4096_h32kv8_d128", "bshd_2x4096_h4kv1_d128", 4),
                           ("bshd_1x16384_h32kv8_d128_w4096", "bshd_1x16384_h4kv1_d128_w4096", 4),
                           ("thd_16seg_h40kv8_d128", "thd_16seg_h5kv1_d128", 5),
                           ("bshd_1x32768_h64kv8_d128_mix", "bshd_1x32768_h8kv1_d128_mix", 8)):
    WORKLOADS[_share] = dataclasses.replace(WORKLOADS[_full], name=_share, num_heads=_hq, num_kv_heads=1)
SHARE_OF = {"bshd_2x4096_h4kv1_d128": "bshd_2x4096_h32kv8_d128",
            "bshd_1x16384_h4kv1_d128_w4096": "bshd_1x16384_h32kv8_d128_w4096",
            "thd_16seg_h5kv1_d128": "thd_16seg_h40kv8_d128",
            "bshd_1x32768_h8kv1_d128_mix": "bshd_1x32768_h64kv8_d128_mix"}


def small_workload(name, *, num_heads, num_kv_heads, head_dim, batch=1, seqlen=0,
                   segment_lengths=(), window=0, use_rope=True, theta=1.0e4, gate_std=1.0,
                   seed=0) -> Workload:
    """A test-sized workload with one layer."""
    return Workload(name, num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    theta=theta, batch=batch, seqlen=seqlen,
                    segment_lengths=tuple(segment_lengths), layers=((window, use_rope),),
                    gate_std=gate_std, seed=seed)


def _stream(seed: int, workload: str, layer: int, tensor: str) -> np.random.Generator:
    key = [int(seed), zlib.crc32(workload.encode()), int(layer), zlib.crc32(tensor.encode())]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def draw_bf16(shape, std, *, seed, workload, layer, tensor) -> np.ndarray:
    """bf16 bit patterns of float32 N(0, std) draws (std is a standard deviation)."""
    rng = _stream(seed, workload, layer, tensor)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _to_bf16_bits(x)


def draw_gain(head_dim, std, *, seed, workload, layer, tensor) -> np.ndarray:
    """Zero-centred gain g ~ N(0, std), float32 holding bf16-representable values."""
    bits = draw_bf16((head_dim,), std, seed=seed, workload=workload, layer=layer, tensor=tensor)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_layer_inputs(w: Workload, layer: int = 0) -> dict:
    """All inputs of one layer of ``w``: q, gate [N,Hq,D]; k, v [N,Hkv,D] (bf16 bits),
    q_gain, k_gain [D] float32, cu_seqlens int32 (THD only), and the layer's
    (window, use_rope)."""
    n, hq, hkv, d = w.tokens, w.num_heads, w.num_kv_heads, w.head_dim
    kw = dict(seed=w.seed, workload=w.name, layer=layer)
    window, use_rope = w.layers[layer]
    out = {
        "q": draw_bf16((n, hq, d), 1.0, tensor="q", **kw),
        "k": draw_bf16((n, hkv, d), 1.0, tensor="k", **kw),
        "v": draw_bf16((n, hkv, d), 1.0, tensor="v", **kw),
        "gate": draw_bf16((n, hq, d), w.gate_std, tensor="gate", **kw),
        "q_gain": draw_gain(d, w.gain_std, tensor="q_gain", **kw),
        "k_gain": draw_gain(d, w.gain_std, tensor="k_gain", **kw),
        "window": int(window),
        "use_rope": bool(use_rope),
    }
    if w.is_thd:
        out["cu_seqlens"] = w.cu_seqlens()
    return out
