"""Python binding of libmuseattn, the MI355X Muse Spark Open attention core.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libmuseattn.so`` (built in-tree by ``decoder_attention_qk_amd._build``).
PyTorch supplies device memory and the current stream.  The functions carry
the C entry points' names; outputs not passed in are allocated with
``torch.empty`` on the input's device.  A non-OK status raises ``MuseError``.
If the library is missing, importing works but every call raises
``RuntimeError`` -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os

__all__ = [
    "MuseError", "AttnParams", "Layout", "library", "library_path", "symbols",
    "muse_rope_cos_sin", "muse_rope_cos_sin_2d", "muse_qk_norm_rope", "muse_qk_norm_rope_table",
    "muse_gqa_attn_fwd", "muse_out_norm_gate", "muse_attn_core_fwd", "muse_attn_fused_fwd", "muse_out_norm_gate_bwd",
    "muse_attn_bwd_delta", "muse_gqa_attn_bwd", "muse_qk_norm_rope_bwd",
    "muse_qk_norm_rope_bwd_workspace_size", "muse_attn_core_bwd", "muse_attn_core_bwd_workspace_size",
    "muse_attn_fwd_workspace_size", "muse_gqa_attn_bwd_workspace_size", "muse_qk_norm_rope_bwd_static",
    "muse_validate_cu_seqlens", "muse_status_string", "muse_version",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmuseattn.so")

MUSE_OK, MUSE_ERR_INVALID_ARG, MUSE_ERR_UNSUPPORTED, MUSE_ERR_DEVICE = 0, 1, 2, 3

# Every symbol include/muse_attn.h declares.
symbols = (
    "muse_rope_cos_sin", "muse_rope_cos_sin_2d", "muse_qk_norm_rope", "muse_qk_norm_rope_table",
    "muse_gqa_attn_fwd", "muse_out_norm_gate", "muse_attn_core_fwd", "muse_attn_fused_fwd", "muse_out_norm_gate_bwd", "muse_attn_bwd_delta",
    "muse_gqa_attn_bwd", "muse_qk_norm_rope_bwd", "muse_qk_norm_rope_bwd_workspace_size",
    "muse_attn_core_bwd", "muse_attn_core_bwd_workspace_size", "muse_attn_fwd_workspace_size",
    "muse_gqa_attn_bwd_workspace_size", "muse_qk_norm_rope_bwd_static", "muse_validate_cu_seqlens",
    "muse_status_string", "muse_last_error", "muse_version",
)


class MuseError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class c_params(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("num_key_value_heads", ctypes.c_int32), ("sliding_window", ctypes.c_int32),
                ("use_rope", ctypes.c_int32), ("upcast_rope", ctypes.c_int32),
                ("scaling", ctypes.c_float), ("query_scale", ctypes.c_float),
                ("qk_eps", ctypes.c_float), ("out_eps", ctypes.c_float),
                ("gain_center", ctypes.c_float), ("bidirectional", ctypes.c_int32),
                ("skip_qk_norm", ctypes.c_int32), ("kv_split", ctypes.c_int32)]


class c_layout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p), ("num_segments", ctypes.c_int32),
                ("total_tokens", ctypes.c_int32), ("max_seqlen", ctypes.c_int32),
                ("position_ids", ctypes.c_void_p), ("attention_mask", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "muse_rope_cos_sin": [ctypes.c_float, _I32, _I32, _P, _P, _P],
    "muse_rope_cos_sin_2d": [ctypes.c_float, _I32, _I32, _I32, _P, _P, _P],
    "muse_qk_norm_rope": [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P],
    "muse_qk_norm_rope_table": [_P, _P, _P, _P, _P, _P, ctypes.c_float, _I32, _P, _P, _P, _P, _P, _P, _P],
    "muse_gqa_attn_fwd": [_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "muse_attn_fwd_workspace_size": [_P, _P, _P],
    "muse_out_norm_gate": [_P, _P, _P, _P, _P, _P, _P],
    "muse_attn_core_fwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "muse_attn_fused_fwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, ctypes.c_size_t, _P],
    "muse_out_norm_gate_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P],
    "muse_attn_bwd_delta": [_P, _P, _P, _P, _P, _P],
    "muse_gqa_attn_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "muse_gqa_attn_bwd_workspace_size": [_P, _P, _P],
    "muse_qk_norm_rope_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _P,
                              ctypes.c_size_t, _P],
    "muse_qk_norm_rope_bwd_workspace_size": [_P, _P, _P],
    "muse_qk_norm_rope_bwd_static": [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _P],
    "muse_attn_core_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                           _P, _P, ctypes.c_size_t, _P],
    "muse_attn_core_bwd_workspace_size": [_P, _P, _P],
    "muse_validate_cu_seqlens": [_P, _I32, _I32, _I32],
    "muse_status_string": [ctypes.c_int],
    "muse_last_error": [],
    "muse_version": [],
}

_lib = None


def library() -> ctypes.CDLL:
    """The loaded libmuseattn (raises RuntimeError when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(library_path)
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name in ("muse_status_string", "muse_last_error",
                                                     "muse_version") else ctypes.c_int
        _lib = lib
    return _lib


def _status_name(status: int) -> str:
    try:
        return library().muse_status_string(status).decode()
    except Exception:  # library unavailable while formatting an error
        return f"status {status}"


def _check(status: int) -> None:
    if status != MUSE_OK:
        raise MuseError(status, library().muse_last_error().decode())


def muse_status_string(status: int) -> str:
    return library().muse_status_string(status).decode()


def muse_version() -> str:
    return library().muse_version().decode()


# ---------------------------------------------------------------- parameters

@dataclasses.dataclass
class AttnParams:
    """One layer's parameters (mirrors ``muse_attn_params``)."""

    head_dim: int
    num_heads: int
    num_key_value_heads: int
    sliding_window: int = 0
    use_rope: bool = True
    upcast_rope: bool = True
    scaling: float | None = None          # None: head_dim ** -0.5
    query_scale: float = 1.0
    qk_eps: float = 1e-6
    out_eps: float = 1e-6
    gain_center: float = 1.0
    bidirectional: bool = False           # packed bidirectional attention (no causal order)
    skip_qk_norm: bool = False            # muse_qk_norm_rope: scale/rotate only (vision attention)
    kv_split: int = 0                     # attention split policy: 0 automatic, 1 never, n >= 2 n parts

    def to_c(self) -> c_params:
        scale = self.head_dim ** -0.5 if self.scaling is None else self.scaling
        return c_params(self.head_dim, self.num_heads, self.num_key_value_heads,
                        int(self.sliding_window or 0), int(bool(self.use_rope)),
                        int(bool(self.upcast_rope)), scale, self.query_scale, self.qk_eps,
                        self.out_eps, self.gain_center, int(bool(self.bidirectional)),
                        int(bool(self.skip_qk_norm)), int(self.kv_split))


@dataclasses.dataclass
class Layout:
    """Token layout (mirrors ``muse_layout``); build with ``bshd`` or ``thd``."""

    batch: int = 0
    seqlen: int = 0
    cu_seqlens: object = None             # torch.int32 device tensor [segments + 1]
    max_seqlen: int = 0
    position_ids: object = None           # optional torch.int32 device tensor [N]
    total_tokens: int | None = None       # THD: cu_seqlens[-1] (read from the device if None)
    attention_mask: object = None         # optional BSHD token validity [batch, seqlen] (bool/uint8)

    @classmethod
    def bshd(cls, batch: int, seqlen: int, position_ids=None, attention_mask=None) -> "Layout":
        return cls(batch=batch, seqlen=seqlen, position_ids=position_ids, attention_mask=attention_mask)

    @classmethod
    def thd(cls, cu_seqlens, max_seqlen: int, position_ids=None, total_tokens=None) -> "Layout":
        return cls(cu_seqlens=cu_seqlens, max_seqlen=int(max_seqlen), position_ids=position_ids,
                   total_tokens=total_tokens)

    @property
    def tokens(self) -> int:
        if self.cu_seqlens is not None:
            return self._total
        return self.batch * self.seqlen

    def to_c(self) -> c_layout:
        if self.cu_seqlens is not None:
            _expect(self.cu_seqlens, "cu_seqlens", "int32")
            nseg = self.cu_seqlens.numel() - 1
            return c_layout(0, 0, self.cu_seqlens.data_ptr(), nseg, self._total, self.max_seqlen,
                            _ptr(self.position_ids, "position_ids", "int32"),
                            _ptr(self.attention_mask, "attention_mask", "mask"))
        return c_layout(self.batch, self.seqlen, None, self.batch, 0, 0,
                        _ptr(self.position_ids, "position_ids", "int32"),
                        _ptr(self.attention_mask, "attention_mask", "mask"))

    @property
    def _total(self) -> int:
        if self.total_tokens is None:
            self.total_tokens = int(self.cu_seqlens[-1].item())
        return self.total_tokens


# ---------------------------------------------------------------- marshalling

def _expect(t, name, dtype):
    import torch
    want = {"bf16": (torch.bfloat16,), "fp32": (torch.float32,), "int32": (torch.int32,),
            "mask": (torch.bool, torch.uint8)}[dtype]
    if t.dtype not in want:
        raise TypeError(f"{name}: expected {' or '.join(map(str, want))}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")


def _ptr(t, name, dtype):
    if t is None:
        return None
    _expect(t, name, dtype)
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _empty(shape, dtype, like):
    import torch
    return torch.empty(shape, dtype=dtype, device=like.device)


def _workspace_size(fn, params, layout) -> int:
    size = ctypes.c_size_t(0)
    p, l = params.to_c(), layout.to_c()
    _check(fn(ctypes.byref(p), ctypes.byref(l), ctypes.byref(size)))
    return size.value


def _ws_ptr(ws):
    if not ws.is_cuda or not ws.is_contiguous():
        raise TypeError("workspace: expected a contiguous GPU tensor")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _fwd_workspace(params, layout, workspace, like):
    """(pointer, bytes) of the caller's forward workspace, or of a fresh one
    when the call needs one and none was given (None, 0 when it needs none)."""
    import torch
    if workspace is not None:
        return _ws_ptr(workspace)
    size = _workspace_size(library().muse_attn_fwd_workspace_size, params, layout)
    if size == 0:
        return None, 0
    return _ws_ptr(torch.empty(size, dtype=torch.uint8, device=like.device))


def muse_rope_cos_sin(theta, head_dim, n_pos, cos_out=None, sin_out=None, *, device=None, stream=None):
    """FP32 cos/sin table [n_pos, head_dim/2]; returns (cos, sin)."""
    import torch
    dev = device if device is not None else (cos_out.device if cos_out is not None else "cuda")
    if cos_out is None:
        cos_out = torch.empty((n_pos, head_dim // 2), dtype=torch.float32, device=dev)
    if sin_out is None:
        sin_out = torch.empty((n_pos, head_dim // 2), dtype=torch.float32, device=dev)
    _check(library().muse_rope_cos_sin(float(theta), int(head_dim), int(n_pos),
                                       _ptr(cos_out, "cos_out", "fp32"),
                                       _ptr(sin_out, "sin_out", "fp32"), _stream(stream)))
    return cos_out, sin_out


def muse_rope_cos_sin_2d(theta, head_dim, grid_h, grid_w, cos_out=None, sin_out=None, *, device=None,
                         stream=None):
    """FP32 2-D cos/sin table [grid_h*grid_w, head_dim/2] of a row-major patch grid."""
    import torch
    dev = device if device is not None else (cos_out.device if cos_out is not None else "cuda")
    n = int(grid_h) * int(grid_w)
    if cos_out is None:
        cos_out = torch.empty((n, head_dim // 2), dtype=torch.float32, device=dev)
    if sin_out is None:
        sin_out = torch.empty((n, head_dim // 2), dtype=torch.float32, device=dev)
    _check(library().muse_rope_cos_sin_2d(float(theta), int(head_dim), int(grid_h), int(grid_w),
                                          _ptr(cos_out, "cos_out", "fp32"),
                                          _ptr(sin_out, "sin_out", "fp32"), _stream(stream)))
    return cos_out, sin_out


def muse_qk_norm_rope(params: AttnParams, layout: Layout, q, k, q_gain=None, k_gain=None, cos=None,
                      sin=None, *, q_out=None, k_out=None, q_rstd=None, k_rstd=None,
                      want_rstd=False, stream=None):
    """Q/K norm + gain + query_scale + RoPE; returns (q_out, k_out, q_rstd, k_rstd)."""
    import torch
    like = q if q is not None else k
    if q is not None and q_out is None:
        q_out = torch.empty_like(q)
    if k is not None and k_out is None:
        k_out = torch.empty_like(k)
    if want_rstd:
        n = like.shape[0]
        if q is not None and q_rstd is None:
            q_rstd = _empty((n, params.num_heads), torch.float32, like)
        if k is not None and k_rstd is None:
            k_rstd = _empty((n, params.num_key_value_heads), torch.float32, like)
    n_pos = cos.shape[0] if cos is not None else 0
    p, l = params.to_c(), layout.to_c()
    _check(library().muse_qk_norm_rope(
        ctypes.byref(p), ctypes.byref(l), _ptr(q, "q", "bf16"), _ptr(k, "k", "bf16"),
        _ptr(q_gain, "q_gain", "fp32"), _ptr(k_gain, "k_gain", "fp32"), _ptr(cos, "cos", "fp32"),
        _ptr(sin, "sin", "fp32"), n_pos, _ptr(q_out, "q_out", "bf16"), _ptr(k_out, "k_out", "bf16"),
        _ptr(q_rstd, "q_rstd", "fp32"), _ptr(k_rstd, "k_rstd", "fp32"), _stream(stream)))
    return q_out, k_out, q_rstd, k_rstd


def muse_qk_norm_rope_table(params: AttnParams, layout: Layout, q, k, q_gain=None, k_gain=None, *,
                            theta: float, n_pos: int, cos_out=None, sin_out=None, q_out=None, k_out=None,
                            q_rstd=None, k_rstd=None, want_rstd=False, stream=None):
    """muse_qk_norm_rope that also builds the RoPE table rows of its tokens'
    positions; returns (q_out, k_out, q_rstd, k_rstd, cos_out, sin_out)."""
    import torch
    like = q if q is not None else k
    if q is not None and q_out is None:
        q_out = torch.empty_like(q)
    if k is not None and k_out is None:
        k_out = torch.empty_like(k)
    if cos_out is None:
        cos_out = _empty((n_pos, params.head_dim // 2), torch.float32, like)
    if sin_out is None:
        sin_out = _empty((n_pos, params.head_dim // 2), torch.float32, like)
    if want_rstd:
        n = like.shape[0]
        if q is not None and q_rstd is None:
            q_rstd = _empty((n, params.num_heads), torch.float32, like)
        if k is not None and k_rstd is None:
            k_rstd = _empty((n, params.num_key_value_heads), torch.float32, like)
    p, l = params.to_c(), layout.to_c()
    _check(library().muse_qk_norm_rope_table(
        ctypes.byref(p), ctypes.byref(l), _ptr(q, "q", "bf16"), _ptr(k, "k", "bf16"),
        _ptr(q_gain, "q_gain", "fp32"), _ptr(k_gain, "k_gain", "fp32"), float(theta), int(n_pos),
        _ptr(cos_out, "cos_out", "fp32"), _ptr(sin_out, "sin_out", "fp32"), _ptr(q_out, "q_out", "bf16"),
        _ptr(k_out, "k_out", "bf16"), _ptr(q_rstd, "q_rstd", "fp32"), _ptr(k_rstd, "k_rstd", "fp32"),
        _stream(stream)))
    return q_out, k_out, q_rstd, k_rstd, cos_out, sin_out


def muse_attn_fwd_workspace_size(params: AttnParams, layout: Layout) -> int:
    """Workspace bytes of the attention forward (the KV split's; 0 without one)."""
    return _workspace_size(library().muse_attn_fwd_workspace_size, params, layout)


def muse_gqa_attn_fwd(params: AttnParams, layout: Layout, q_hat, k_hat, v, *, o=None, lse=None,
                      want_lse=False, workspace=None, stream=None):
    """Causal GQA attention; returns (o, lse)."""
    import torch
    if o is None:
        o = torch.empty_like(q_hat)
    if want_lse and lse is None:
        lse = _empty(q_hat.shape[:2], torch.float32, q_hat)
    wp, wb = _fwd_workspace(params, layout, workspace, q_hat)
    p, l = params.to_c(), layout.to_c()
    _check(library().muse_gqa_attn_fwd(
        ctypes.byref(p), ctypes.byref(l), _ptr(q_hat, "q_hat", "bf16"), _ptr(k_hat, "k_hat", "bf16"),
        _ptr(v, "v", "bf16"), _ptr(o, "o", "bf16"), _ptr(lse, "lse", "fp32"), wp, wb, _stream(stream)))
    return o, lse


def muse_out_norm_gate(params: AttnParams, layout: Layout, o, gate, *, out=None, o_rstd=None,
                       want_rstd=False, stream=None):
    """Output RMSNorm x sigmoid(gate); returns (out, o_rstd)."""
    import torch
    if out is None:
        out = torch.empty_like(o)
    if want_rstd and o_rstd is None:
        o_rstd = _empty(o.shape[:2], torch.float32, o)
    p, l = params.to_c(), layout.to_c()
    _check(library().muse_out_norm_gate(
        ctypes.byref(p), ctypes.byref(l), _ptr(o, "o", "bf16"), _ptr(gate, "gate", "bf16"),
        _ptr(out, "out", "bf16"), _ptr(o_rstd, "o_rstd", "fp32"), _stream(stream)))
    return out, o_rstd


def muse_attn_core_fwd(params: AttnParams, layout: Layout, q, k, v, gate, q_gain=None, k_gain=None,
                       cos=None, sin=None, *, k_hat_out=None, out=None, lse=None, want_lse=False,
                       workspace=None, stream=None):
    """The fused core; returns (out, k_hat_out, lse)."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    if k_hat_out is None:
        k_hat_out = torch.empty_like(k)
    if want_lse and lse is None:
        lse = _empty(q.shape[:2], torch.float32, q)
    n_pos = cos.shape[0] if cos is not None else 0
    wp, wb = _fwd_workspace(params, layout, workspace, q)
    p, l = params.to_c(), layout.to_c()
    _check(library().muse_attn_core_fwd(
        ctypes.byref(p), ctypes.byref(l), _ptr(q, "q", "bf16"), _ptr(k, "k", "bf16"),
        _ptr(v, "v", "bf16"), _ptr(gate, "gate", "bf16"), _ptr(q_gain, "q_gain", "fp32"),
        _ptr(k_gain, "k_gain", "fp32"), _ptr(cos, "cos", "fp32"), _ptr(sin, "sin", "fp32"), n_pos,
        _ptr(k_hat_out, "k_hat_out", "bf16"), _ptr(out, "out", "bf16"), _ptr(lse, "lse", "fp32"),
        wp, wb, _stream(stream)))
    return out, k_hat_out, lse


def muse_attn_fused_fwd(params: AttnParams, layout: Layout, q, k_hat, v, gate, q_gain=None, cos=None,
                        sin=None, *, out=None, lse=None, want_lse=False, workspace=None, stream=None):
    """Fused attention on already-normalised keys; returns (out, lse)."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = _empty(q.shape[:2], torch.float32, q)
    n_pos = cos.shape[0] if cos is not None else 0
    wp, wb = _fwd_workspace(params, layout, workspace, q)
    p, l = params.to_c(), layout.to_c()
    _check(library().muse_attn_fused_fwd(
        ctypes.byref(p), ctypes.byref(l), _ptr(q, "q", "bf16"), _ptr(k_hat, "k_hat", "bf16"),
        _ptr(v, "v", "bf16"), _ptr(gate, "gate", "bf16"), _ptr(q_gain, "q_gain", "fp32"),
        _ptr(cos, "cos", "fp32"), _ptr(sin, "sin", "fp32"), n_pos, _ptr(out, "out", "bf16"),
        _ptr(lse, "lse", "fp32"), wp, wb, _stream(stream)))
    return out, lse


# ---------------------------------------------------------------- backward

def _workspace(fn, params, layout, workspace, like):
    """A caller's workspace, or a fresh one of the size the library reports."""
    import torch
    size = _workspace_size(fn, params, layout)
    if workspace is None:
        workspace = torch.empty(max(1, size), dtype=torch.uint8, device=like.device)
    return workspace, size


def muse_out_norm_gate_bwd(params: AttnParams, layout: Layout, o, gate, dout, *, d_o=None, dgate=None,
                           delta=None, stream=None):
    """Backward of the output norm + gate; returns (d_o, dgate, delta)."""
    import torch
    d_o = torch.empty_like(o) if d_o is None else d_o
    dgate = torch.empty_like(o) if dgate is None else dgate
    delta = _empty(o.shape[:2], torch.float32, o) if delta is None else delta
    p, l = params.to_c(), layout.to_c()
    _check(library().muse_out_norm_gate_bwd(
        ctypes.byref(p), ctypes.byref(l), _ptr(o, "o", "bf16"), _ptr(gate, "gate", "bf16"),
        _ptr(dout, "dout", "bf16"), _ptr(d_o, "d_o", "bf16"), _ptr(dgate, "dgate", "bf16"),
        _ptr(delta, "delta", "fp32"), _stream(stream)))
    return d_o, dgate, delta


def muse_attn_bwd_delta(params: AttnParams, layout: Layout, o, d_o, *, delta=None, stream=None):
    """delta = rowsum(d_o * o) [N, Hq] fp32."""
    import torch
    delta = _empty(o.shape[:2], torch.float32, o) if delta is None else delta
    p, l = params.to_c(), layout.to_c()
    _check(library().muse_attn_bwd_delta(ctypes.byref(p), ctypes.byref(l), _ptr(o, "o", "bf16"),
                                         _ptr(d_o, "d_o", "bf16"), _ptr(delta, "delta", "fp32"),
                                         _stream(stream)))
    return delta


def muse_gqa_attn_bwd_workspace_size(params: AttnParams, layout: Layout) -> int:
    """Workspace bytes of the attention backward (its splits'; 0 without one)."""
    return _workspace_size(library().muse_gqa_attn_bwd_workspace_size, params, layout)


def muse_gqa_attn_bwd(params: AttnParams, layout: Layout, q_hat, k_hat, v, d_o, lse, delta, *,
                      dq_hat=None, dk_hat=None, dv=None, workspace=None, stream=None):
    """Attention backward; returns (dq_hat, dk_hat, dv)."""
    import torch
    dq_hat = torch.empty_like(q_hat) if dq_hat is None else dq_hat
    dk_hat = torch.empty_like(k_hat) if dk_hat is None else dk_hat
    dv = torch.empty_like(v) if dv is None else dv
    workspace, _ = _workspace(library().muse_gqa_attn_bwd_workspace_size, params, layout, workspace, q_hat)
    wp, wb = _ws_ptr(workspace)
    p, l = params.to_c(), layout.to_c()
    _check(library().muse_gqa_attn_bwd(
        ctypes.byref(p), ctypes.byref(l), _ptr(q_hat, "q_hat", "bf16"), _ptr(k_hat, "k_hat", "bf16"),
        _ptr(v, "v", "bf16"), _ptr(d_o, "d_o", "bf16"), _ptr(lse, "lse", "fp32"),
        _ptr(delta, "delta", "fp32"), _ptr(dq_hat, "dq_hat", "bf16"), _ptr(dk_hat, "dk_hat", "bf16"),
        _ptr(dv, "dv", "bf16"), wp, wb, _stream(stream)))
    return dq_hat, dk_hat, dv


def muse_qk_norm_rope_bwd(params: AttnParams, layout: Layout, q, k, q_gain, k_gain, cos, sin, dq_hat,
                          dk_hat, *, dq=None, dk=None, dq_gain=None, dk_gain=None, workspace=None,
                          stream=None):
    """Backward of the Q/K norm + RoPE; returns (dq, dk, dq_gain, dk_gain)."""
    import torch
    like = q if q is not None else k
    if q is not None and dq is None:
        dq = torch.empty_like(q)
    if k is not None and dk is None:
        dk = torch.empty_like(k)
    if q_gain is not None and dq_gain is None:
        dq_gain = torch.empty_like(q_gain)
    if k_gain is not None and dk_gain is None:
        dk_gain = torch.empty_like(k_gain)
    workspace, _ = _workspace(library().muse_qk_norm_rope_bwd_workspace_size, params, layout, workspace, like)
    wp, wb = _ws_ptr(workspace)
    n_pos = cos.shape[0] if cos is not None else 0
    p, l = params.to_c(), layout.to_c()
    _check(library().muse_qk_norm_rope_bwd(
        ctypes.byref(p), ctypes.byref(l), _ptr(q, "q", "bf16"), _ptr(k, "k", "bf16"),
        _ptr(q_gain, "q_gain", "fp32"), _ptr(k_gain, "k_gain", "fp32"), _ptr(cos, "cos", "fp32"),
        _ptr(sin, "sin", "fp32"), n_pos, _ptr(dq_hat, "dq_hat", "bf16"), _ptr(dk_hat, "dk_hat", "bf16"),
        _ptr(dq, "dq", "bf16"), _ptr(dk, "dk", "bf16"), _ptr(dq_gain, "dq_gain", "fp32"),
        _ptr(dk_gain, "dk_gain", "fp32"), wp, wb, _stream(stream)))
    return dq, dk, dq_gain, dk_gain


def muse_qk_norm_rope_bwd_static(params: AttnParams, layout: Layout, q, k, q_gain, k_gain, cos, sin, dq_hat,
                                 dk_hat, *, dq=None, dk=None, dq_gain=None, dk_gain=None, stream=None):
    """muse_qk_norm_rope_bwd with the library's static scratch instead of a
    workspace (the C call allocates nothing; outputs not passed in are
    allocated here); returns (dq, dk, dq_gain, dk_gain)."""
    import torch
    if q is not None and dq is None:
        dq = torch.empty_like(q)
    if k is not None and dk is None:
        dk = torch.empty_like(k)
    if q_gain is not None and dq_gain is None:
        dq_gain = torch.empty_like(q_gain)
    if k_gain is not None and dk_gain is None:
        dk_gain = torch.empty_like(k_gain)
    n_pos = cos.shape[0] if cos is not None else 0
    p, l = params.to_c(), layout.to_c()
    _check(library().muse_qk_norm_rope_bwd_static(
        ctypes.byref(p), ctypes.byref(l), _ptr(q, "q", "bf16"), _ptr(k, "k", "bf16"),
        _ptr(q_gain, "q_gain", "fp32"), _ptr(k_gain, "k_gain", "fp32"), _ptr(cos, "cos", "fp32"),
        _ptr(sin, "sin", "fp32"), n_pos, _ptr(dq_hat, "dq_hat", "bf16"), _ptr(dk_hat, "dk_hat", "bf16"),
        _ptr(dq, "dq", "bf16"), _ptr(dk, "dk", "bf16"), _ptr(dq_gain, "dq_gain", "fp32"),
        _ptr(dk_gain, "dk_gain", "fp32"), _stream(stream)))
    return dq, dk, dq_gain, dk_gain


def muse_attn_core_bwd(params: AttnParams, layout: Layout, q, k, v, gate, dout, q_gain=None, k_gain=None,
                       cos=None, sin=None, o=None, lse=None, *, dq=None, dk=None, dv=None, dgate=None,
                       dq_gain=None, dk_gain=None, workspace=None, stream=None):
    """Backward of the whole core; returns (dq, dk, dv, dgate, dq_gain, dk_gain).

    o and lse from the forward (attention output before the output norm, and
    its LSE) may be omitted together: they are recomputed."""
    import torch
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dgate = torch.empty_like(gate) if dgate is None else dgate
    if q_gain is not None and dq_gain is None:
        dq_gain = torch.empty_like(q_gain)
    if k_gain is not None and dk_gain is None:
        dk_gain = torch.empty_like(k_gain)
    workspace, _ = _workspace(library().muse_attn_core_bwd_workspace_size, params, layout, workspace, q)
    wp, wb = _ws_ptr(workspace)
    n_pos = cos.shape[0] if cos is not None else 0
    p, l = params.to_c(), layout.to_c()
    _check(library().muse_attn_core_bwd(
        ctypes.byref(p), ctypes.byref(l), _ptr(q, "q", "bf16"), _ptr(k, "k", "bf16"), _ptr(v, "v", "bf16"),
        _ptr(gate, "gate", "bf16"), _ptr(q_gain, "q_gain", "fp32"), _ptr(k_gain, "k_gain", "fp32"),
        _ptr(cos, "cos", "fp32"), _ptr(sin, "sin", "fp32"), n_pos, _ptr(o, "o", "bf16"),
        _ptr(lse, "lse", "fp32"), _ptr(dout, "dout", "bf16"), _ptr(dq, "dq", "bf16"), _ptr(dk, "dk", "bf16"),
        _ptr(dv, "dv", "bf16"), _ptr(dgate, "dgate", "bf16"), _ptr(dq_gain, "dq_gain", "fp32"),
        _ptr(dk_gain, "dk_gain", "fp32"), wp, wb, _stream(stream)))
    return dq, dk, dv, dgate, dq_gain, dk_gain


def muse_validate_cu_seqlens(cu_seqlens, num_segments, total_tokens, max_seqlen) -> int:
    """Pure host check of packed boundaries (a sequence of ints); returns the status."""
    arr = (ctypes.c_int32 * len(cu_seqlens))(*[int(x) for x in cu_seqlens])
    return library().muse_validate_cu_seqlens(ctypes.cast(arr, ctypes.c_void_p), int(num_segments),
                                              int(total_tokens), int(max_seqlen))
