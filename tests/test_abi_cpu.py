"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before enqueuing
anything.  Every call here fails host validation by construction (fake
pointers are never dereferenced), so no kernel is launched."""

import ctypes
import os
import re
import subprocess

import pytest

import decoder_attention_qk_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muse_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muse_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(m.symbols) == _declared_functions()


def test_library_exports_every_declared_symbol():
    lib = m.library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", m.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (muse_[a-z0-9_]+)$", out, flags=re.M))
    assert set(_declared_functions()) <= exported


def test_status_strings_and_version():
    assert m.muse_status_string(0) == "MUSE_OK"
    assert m.muse_status_string(1) == "MUSE_ERR_INVALID_ARG"
    assert m.muse_status_string(2) == "MUSE_ERR_UNSUPPORTED"
    assert m.muse_status_string(3) == "MUSE_ERR_DEVICE"
    assert re.fullmatch(r"\d+\.\d+\.\d+", m.muse_version())


@pytest.mark.parametrize("cu,nseg,total,maxlen,ok", [
    ([0, 3, 5], 2, 5, 3, True),
    ([0, 0, 4, 4], 3, 4, 4, True),              # empty documents are allowed
    ([0], 0, 0, 0, False),                      # no segment
    ([1, 3, 5], 2, 5, 3, False),                # must start at 0
    ([0, 3, 2], 2, 2, 3, False),                # decreasing
    ([0, 3, 5], 2, 6, 3, False),                # last != total
    ([0, 3, 8], 2, 8, 4, False),                # a segment longer than max_seqlen
])
def test_validate_cu_seqlens(cu, nseg, total, maxlen, ok):
    status = m.muse_validate_cu_seqlens(cu, nseg, total, maxlen)
    assert (status == 0) == ok
    if not ok:
        assert status == 1 and m.library().muse_last_error().decode()


FAKE = 0x7F0000000000   # a host-side stand-in address; validation never dereferences it


def _params(**kw):
    p = dict(head_dim=128, num_heads=8, num_key_value_heads=2, sliding_window=0, use_rope=1,
             upcast_rope=1, scaling=128 ** -0.5, query_scale=1.0, qk_eps=1e-6, out_eps=1e-6,
             gain_center=1.0)
    p.update(kw)
    return m.c_params(**p)


def _bshd(batch=1, seqlen=16):
    return m.c_layout(batch, seqlen, None, batch, 0, 0, None)


def _attn(p, lay, q=FAKE, k=FAKE + (1 << 24), v=FAKE + (2 << 24), o=FAKE + (3 << 24), lse=None, ws=None,
          wsb=0):
    return m.library().muse_gqa_attn_fwd(ctypes.byref(p) if p is not None else None,
                                         ctypes.byref(lay) if lay is not None else None,
                                         q, k, v, o, lse, ws, wsb, None)


def test_null_params_and_layout():
    assert _attn(None, _bshd()) == 1
    assert _attn(_params(), None) == 1


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=0), 1), (dict(head_dim=127), 1), (dict(num_heads=0), 1),
    (dict(num_heads=6, num_key_value_heads=4), 1), (dict(scaling=0.0), 1),
    (dict(scaling=float("nan")), 1), (dict(qk_eps=-1.0), 1), (dict(out_eps=float("inf")), 1),
    (dict(query_scale=float("inf")), 1), (dict(gain_center=float("nan")), 1),
    (dict(bidirectional=1, sliding_window=8), 1), (dict(kv_split=-1), 1),
    (dict(head_dim=96), 2), (dict(head_dim=256), 2),
])
def test_bad_params(kw, status):
    assert _attn(_params(**kw), _bshd()) == status
    assert m.library().muse_last_error().decode()


def test_bad_layouts():
    assert _attn(_params(), _bshd(-1, 4)) == 1
    thd = m.c_layout(0, 0, FAKE + (9 << 24), 0, 10, 10, None)       # no segment
    assert _attn(_params(), thd) == 1
    thd = m.c_layout(0, 0, FAKE + (9 << 24), 2, 10, 11, None)       # max_seqlen > total
    assert _attn(_params(), thd) == 1
    thd = m.c_layout(0, 0, FAKE + (9 << 24), 2, 10, 0, None)        # max_seqlen 0 with tokens
    assert _attn(_params(), thd) == 1


def test_missing_and_overlapping_buffers():
    assert _attn(_params(), _bshd(), q=None) == 1
    assert _attn(_params(), _bshd(), o=None) == 1
    # o overlapping q (same base) and lse overlapping o
    assert _attn(_params(), _bshd(), o=FAKE) == 1
    assert "overlaps" in m.library().muse_last_error().decode()
    assert _attn(_params(), _bshd(), lse=FAKE + (3 << 24) + 64) == 1


def test_misaligned_buffers():
    # bf16 tensors need 16-byte alignment, per-row fp32 outputs 4-byte
    assert _attn(_params(), _bshd(), q=FAKE + 2) == 1
    assert "aligned" in m.library().muse_last_error().decode()
    assert _attn(_params(), _bshd(), o=FAKE + (3 << 24) + 8) == 1
    assert _attn(_params(), _bshd(), lse=FAKE + (4 << 24) + 2) == 1
    assert "aligned" in m.library().muse_last_error().decode()


def test_qk_norm_rope_argument_rules():
    lib = m.library()
    p, lay = _params(), _bshd()
    base = [FAKE, FAKE + (1 << 24), None, None, FAKE + (2 << 24), FAKE + (3 << 24), 16,
            FAKE + (4 << 24), FAKE + (5 << 24), None, None]

    def call(**over):
        a = dict(zip(["q", "k", "qg", "kg", "cos", "sin", "npos", "qo", "ko", "qr", "kr"], base))
        a.update(over)
        return lib.muse_qk_norm_rope(ctypes.byref(p), ctypes.byref(lay), a["q"], a["k"], a["qg"],
                                     a["kg"], a["cos"], a["sin"], a["npos"], a["qo"], a["ko"],
                                     a["qr"], a["kr"], None)
    assert call(q=None, qo=None, k=None, ko=None) == 1     # nothing to do
    assert call(qo=None) == 1                              # input without output
    assert call(cos=None) == 1                             # rope without table
    assert call(npos=8) == 1                               # table shorter than the row
    assert call(qo=FAKE + 100) == 1                        # output overlaps input


def test_qk_norm_rope_table_argument_rules():
    lib = m.library()
    lay = _bshd()
    base = dict(q=FAKE, k=FAKE + (1 << 24), qg=None, kg=None, theta=1e4, npos=16, cos=FAKE + (2 << 24),
                sin=FAKE + (3 << 24), qo=FAKE + (4 << 24), ko=FAKE + (5 << 24), qr=None, kr=None)

    def call(p=None, **over):
        a = dict(base)
        a.update(over)
        return lib.muse_qk_norm_rope_table(ctypes.byref(p or _params()), ctypes.byref(lay), a["q"], a["k"],
                                           a["qg"], a["kg"], a["theta"], a["npos"], a["cos"], a["sin"],
                                           a["qo"], a["ko"], a["qr"], a["kr"], None)
    assert call(p=_params(use_rope=0)) == 1                # the table is a RoPE table
    assert call(theta=0.0) == 1
    assert call(theta=float("nan")) == 1
    assert call(cos=None) == 1
    assert call(npos=8) == 1                               # table shorter than the row
    assert call(cos=FAKE + 100) == 1                       # table output overlaps input q
    assert call(sin=FAKE + (2 << 24) + 64) == 1            # the two tables overlap
    assert call(ko=FAKE + (2 << 24)) == 1                  # k_out overlaps cos_out
    assert call(q=None, qo=None, k=None, ko=None) == 1     # nothing to do


def test_rope_table_argument_rules():
    lib = m.library()
    assert lib.muse_rope_cos_sin(0.0, 64, 4, FAKE, FAKE + 4096, None) == 1
    assert lib.muse_rope_cos_sin(1e4, 63, 4, FAKE, FAKE + 4096, None) == 1
    assert lib.muse_rope_cos_sin(1e4, 64, -1, FAKE, FAKE + 4096, None) == 1
    assert lib.muse_rope_cos_sin(1e4, 64, 4, None, FAKE, None) == 1
    assert lib.muse_rope_cos_sin(1e4, 64, 4, FAKE, FAKE + 64, None) == 1   # overlapping outputs


def test_rope_table_2d_argument_rules():
    lib = m.library()
    assert lib.muse_rope_cos_sin_2d(0.0, 64, 2, 2, FAKE, FAKE + 4096, None) == 1
    assert lib.muse_rope_cos_sin_2d(1e4, 62, 2, 2, FAKE, FAKE + 4096, None) == 1   # D % 4 != 0
    assert lib.muse_rope_cos_sin_2d(1e4, 64, -1, 2, FAKE, FAKE + 4096, None) == 1
    assert lib.muse_rope_cos_sin_2d(1e4, 64, 2, -1, FAKE, FAKE + 4096, None) == 1
    assert lib.muse_rope_cos_sin_2d(1e4, 64, 2, 2, None, FAKE, None) == 1
    assert lib.muse_rope_cos_sin_2d(1e4, 64, 2, 2, FAKE, FAKE + 64, None) == 1   # overlapping outputs
    assert lib.muse_rope_cos_sin_2d(1e4, 64, 1 << 16, 1 << 16, FAKE, FAKE + 4096, None) == 1
    assert lib.muse_rope_cos_sin_2d(1e4, 64, 0, 7, None, None, None) == 0         # empty grid: no-op


def test_skip_qk_norm_rules():
    lib = m.library()
    p, lay = _params(skip_qk_norm=1), _bshd()
    qo, ko = FAKE + (4 << 24), FAKE + (5 << 24)

    def qk(qg=None, qr=None):
        return lib.muse_qk_norm_rope(ctypes.byref(p), ctypes.byref(lay), FAKE, FAKE + (1 << 24), qg, None,
                                     FAKE + (2 << 24), FAKE + (3 << 24), 16, qo, ko, qr, None, None)
    assert qk(qg=FAKE + (6 << 24)) == 1                    # no gain without the norm
    assert qk(qr=FAKE + (7 << 24)) == 1                    # no rstd without the norm
    # the fused core normalises the query in its prologue
    st = lib.muse_attn_fused_fwd(ctypes.byref(p), ctypes.byref(lay), FAKE, FAKE + (1 << 24),
                                 FAKE + (2 << 24), FAKE + (3 << 24), None, FAKE + (4 << 24),
                                 FAKE + (5 << 24), 16, FAKE + (6 << 24), None, None, 0, None)
    assert st == 2


def test_attention_mask_rules():
    # a key-validity mask is for BSHD only; it is an input (no output may overlap it)
    thd = m.c_layout(0, 0, FAKE + (9 << 24), 2, 10, 5, None, FAKE + (10 << 24))
    assert _attn(_params(), thd) == 1
    assert "THD" in m.library().muse_last_error().decode()
    lay = m.c_layout(1, 16, None, 1, 0, 0, None, FAKE + (3 << 24) + 3)   # inside o, odd address is fine
    assert _attn(_params(), lay) == 1
    assert "overlaps" in m.library().muse_last_error().decode()


def test_backward_argument_rules():
    lib = m.library()
    p, lay = _params(), _bshd(1, 16)
    size = ctypes.c_size_t(0)
    assert lib.muse_attn_core_bwd_workspace_size(ctypes.byref(p), ctypes.byref(lay), ctypes.byref(size)) == 0
    # q_hat, k_hat, o, lse, d_o, delta, dq_hat, dk_hat and the gain partials
    assert size.value >= 16 * 8 * 128 * 2 * 4 + 16 * 2 * 128 * 2 * 2
    need = size.value
    assert lib.muse_qk_norm_rope_bwd_workspace_size(ctypes.byref(p), ctypes.byref(lay), ctypes.byref(size)) == 0
    assert 0 < size.value < need

    A = [FAKE + (i << 24) for i in range(24)]

    def core(pp=p, o=None, lse=None, qg=None, dqg=None, ws=A[20], wsb=need):
        return lib.muse_attn_core_bwd(ctypes.byref(pp), ctypes.byref(lay), A[0], A[1], A[2], A[3], qg, None,
                                      A[4], A[5], 16, o, lse, A[6], A[7], A[8], A[9], A[10], dqg, None, ws,
                                      wsb, None)
    assert core(o=A[11]) == 1                              # o without lse
    assert core(qg=A[12]) == 1                             # a gain without its gradient
    assert core(ws=None) == 1                              # no workspace
    assert core(wsb=need - 1) == 1                         # too small
    assert "workspace" in lib.muse_last_error().decode()
    assert core(ws=A[20] + 8) == 1                         # misaligned workspace
    assert core(pp=_params(upcast_rope=0), ws=None) == 1   # the Q/K-dtype rotation passes the mode checks
    assert core(pp=_params(skip_qk_norm=1)) == 2
    # the attention backward needs every tensor
    st = lib.muse_gqa_attn_bwd(ctypes.byref(p), ctypes.byref(lay), A[0], A[1], A[2], A[3], A[4], None,
                               A[6], A[7], A[8], None, 0, None)
    assert st == 1
    # and the Q/K backward takes a tensor's three buffers together
    st = lib.muse_qk_norm_rope_bwd(ctypes.byref(p), ctypes.byref(lay), A[0], None, None, None, A[4], A[5], 16,
                                   None, None, A[7], None, None, None, None, 0, None)
    assert st == 1


def _size(fn, p, lay):
    size = ctypes.c_size_t(12345)
    assert fn(ctypes.byref(p), ctypes.byref(lay), ctypes.byref(size)) == 0
    return size.value


def test_split_workspace_rules():
    """The KV split keeps its partial slots and counters in the caller's
    workspace: a forced split (kv_split >= 2) needs one, sized by the query,
    and a call without it, with too little, misaligned or overlapping an
    input is rejected before any launch."""
    lib = m.library()
    lay = _bshd(1, 1000)                                   # 8 query blocks, up to 16 key tiles each
    whole = _size(lib.muse_attn_fwd_workspace_size, _params(kv_split=1), lay)
    assert whole == 0
    p = _params(kv_split=3)
    need = _size(lib.muse_attn_fwd_workspace_size, p, lay)
    # counters (items x 4 waves) plus a slot per (item, part, wave) of 130 x 64 floats
    items = 8 * 2
    assert need >= items * 3 * 4 * (128 // 32 * 16 + 2) * 64 * 4 + items * 4 * 4
    ws = FAKE + (8 << 24)
    assert _attn(p, lay, ws=None, wsb=0) == 1
    assert "workspace" in lib.muse_last_error().decode()
    assert _attn(p, lay, ws=ws, wsb=need - 1) == 1
    assert _attn(p, lay, ws=ws + 8, wsb=need) == 1
    assert "aligned" in lib.muse_last_error().decode()
    assert _attn(p, lay, ws=FAKE + (1 << 24) - 256, wsb=need) == 1   # overlaps k
    assert "overlaps" in lib.muse_last_error().decode()
    # the fused entry points take the same workspace
    st = lib.muse_attn_fused_fwd(ctypes.byref(p), ctypes.byref(lay), FAKE, FAKE + (1 << 24), FAKE + (2 << 24),
                                 FAKE + (3 << 24), None, FAKE + (4 << 24), FAKE + (5 << 24), 1000,
                                 FAKE + (6 << 24), None, None, 0, None)
    assert st == 1 and "workspace" in lib.muse_last_error().decode()
    st = lib.muse_attn_core_fwd(ctypes.byref(p), ctypes.byref(lay), FAKE, FAKE + (1 << 24), FAKE + (2 << 24),
                                FAKE + (3 << 24), None, None, FAKE + (4 << 24), FAKE + (5 << 24), 1000,
                                FAKE + (7 << 24), FAKE + (6 << 24), None, ws, need - 16, None)
    assert st == 1 and "workspace" in lib.muse_last_error().decode()


def test_backward_split_workspace_rules():
    lib = m.library()
    lay = _bshd(1, 1000)
    assert _size(lib.muse_gqa_attn_bwd_workspace_size, _params(kv_split=1), lay) == 0
    p = _params(kv_split=4)
    need = _size(lib.muse_gqa_attn_bwd_workspace_size, p, lay)
    assert need > 0
    A = [FAKE + (i << 24) for i in range(12)]

    def bwd(ws, wsb):
        return lib.muse_gqa_attn_bwd(ctypes.byref(p), ctypes.byref(lay), A[0], A[1], A[2], A[3], A[4], A[5],
                                     A[6], A[7], A[8], ws, wsb, None)
    assert bwd(None, 0) == 1
    assert bwd(A[9], need - 1) == 1
    assert "workspace" in lib.muse_last_error().decode()
    # the core backward's workspace holds the split region besides its tensors
    core_split = _size(lib.muse_attn_core_bwd_workspace_size, p, lay)
    core_whole = _size(lib.muse_attn_core_bwd_workspace_size, _params(kv_split=1), lay)
    assert core_split >= core_whole + need


def test_sources_allocate_nothing():
    """No allocation anywhere in the library's sources, and the only
    synchronisation is the opt-in debug check's."""
    csrc = os.path.join(ROOT, "decoder_attention_qk_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        text = re.sub(r"//[^\n]*", "", open(os.path.join(csrc, name)).read())
        for call in ("hipMalloc", "hipFree", "hipHostMalloc", "hipMallocAsync", "hipExtMallocWithFlags",
                     "malloc(", "hipHostRegister"):
            assert call not in text, (name, call)
        if name != "debug_check.cpp":
            for call in ("hipStreamSynchronize", "hipDeviceSynchronize", "hipEventSynchronize", "hipMemcpy"):
                assert call not in text, (name, call)


def test_static_qk_bwd_argument_rules():
    """The allocation-free Q/K backward validates like the workspace one
    (these calls fail before any device work)."""
    lib = m.library()
    p, lay = _params(), _bshd(1, 16)
    A = [FAKE + (i << 24) for i in range(12)]

    def call(q=A[0], dqh=A[1], dq=A[2], qg=None, dqg=None, pp=p):
        return lib.muse_qk_norm_rope_bwd_static(ctypes.byref(pp), ctypes.byref(lay), q, None, qg, None, A[4],
                                                A[5], 16, dqh, None, dq, None, dqg, None, None)
    assert call(dq=None) == 1                              # a tensor without its gradient output
    assert call(qg=A[6]) == 1                              # a gain without its gradient
    assert call(pp=_params(head_dim=96)) == 2
    assert call(pp=_params(kv_split=-2)) == 1
