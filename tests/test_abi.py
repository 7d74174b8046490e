"""The C ABI on the host, with no GPU: the library loads, exports every symbol
include/gdn.h declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

import frame_wise_gated_fwd_amd as F
from frame_wise_gated_fwd_amd._lib import SIGNATURES, Shape

INCLUDE = os.path.join(os.path.dirname(__file__), "..", "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))

OK, NULLPTR, SHAPE, DTYPE, UNSUP_D, WORKSPACE, ALIAS, HIP, VALUE, TIMEOUT = range(10)
F32, BF16 = 0, 1


def declared_functions():
    txt = "".join(open(h).read() for h in HEADERS)
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", txt)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(SIGNATURES)


def test_library_exports_every_declared_symbol():
    L = F.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.gdn_abi_version() == 3


def test_status_strings():
    L = F.lib()
    for s in range(11):
        assert L.gdn_status_str(s) != b"unknown status"
    assert L.gdn_status_str(99) == b"unknown status"


@pytest.mark.parametrize("D,ok", [(16, 1), (32, 1), (64, 1), (112, 1), (128, 1), (0, 0), (8, 0),
                                  (100, 0), (144, 0), (256, 0)])
def test_supported_head_dims(D, ok):
    assert F.lib().gdn_supports_d(D) == ok


def _shape(B=1, H=2, T=3, S=40, D=128):
    return Shape(B, H, T, S, D)


def test_path_selection():
    L = F.lib()
    assert L.gdn_path(ctypes.byref(_shape(1, 16, 961, 880, 128)), BF16) == 2
    assert L.gdn_path(ctypes.byref(_shape(4, 16, 961, 880, 128)), BF16) == 2
    assert L.gdn_path(ctypes.byref(_shape(1, 16, 32, 880, 128)), BF16) == 1
    assert L.gdn_path(ctypes.byref(_shape(1, 16, 1, 880, 128)), BF16) == 3
    assert L.gdn_path(ctypes.byref(_shape(5, 16, 1, 1, 128)), BF16) == 3
    assert L.gdn_path(ctypes.byref(_shape(1, 16, 2, 880, 128)), BF16) == 1
    assert L.gdn_path(ctypes.byref(_shape(1, 16, 1, 880, 64)), BF16) == 0
    assert L.gdn_path(ctypes.byref(_shape(1, 16, 1, 880, 128)), F32) == 0
    assert L.gdn_path(ctypes.byref(_shape(1, 16, 33, 880, 128)), BF16) == 2
    assert L.gdn_path(ctypes.byref(_shape(1, 16, 64, 880, 128)), BF16) == 2
    assert L.gdn_path(ctypes.byref(_shape(1, 16, 961, 880, 128)), F32) == 0
    assert L.gdn_path(ctypes.byref(_shape(1, 2, 8, 16, 64)), BF16) == 0
    assert L.gdn_path(ctypes.byref(_shape(D=100)), BF16) == -1
    assert L.gdn_path(None, BF16) == -1


def test_fused_switch_selects_path():
    L = F.lib()
    s = _shape(1, 16, 961, 880, 128)
    prev = L.gdn_set_fused(0)
    try:
        assert L.gdn_path(ctypes.byref(s), BF16) == 1
        assert L.gdn_set_fused(1) == 0
        assert L.gdn_path(ctypes.byref(s), BF16) == 2
        assert F.set_fused(False) is True
        assert L.gdn_path(ctypes.byref(s), BF16) == 1
    finally:
        L.gdn_set_fused(prev)


def test_single_frame_switch_selects_path():
    L = F.lib()
    s = _shape(1, 16, 1, 880, 128)
    prev = L.gdn_set_single_frame(0)
    prev_fused = L.gdn_set_fused(1)
    try:
        assert L.gdn_path(ctypes.byref(s), BF16) == 1
        assert L.gdn_set_single_frame(1) == 0
        assert L.gdn_path(ctypes.byref(s), BF16) == 3
        assert F.set_single_frame(False) is True
        assert L.gdn_path(ctypes.byref(s), BF16) == 1
        # the fused switch leaves single frames alone
        assert F.set_fused(False) is True
        assert F.set_single_frame(True) is False
        assert L.gdn_path(ctypes.byref(s), BF16) == 3
    finally:
        L.gdn_set_single_frame(prev)
        L.gdn_set_fused(prev_fused)


def _frame_bytes(H, S, B=1):
    """The single-frame kernel runs without a workspace; up to 16 heads it
    asks for one that holds, per 16-row block (8 per head), a 128-byte pair
    word and two halves' partial sums of 8 KiB, so that the block's token
    halves can go to two workgroups."""
    heads = B * H
    if heads == 0 or heads > 16:
        return 0
    pairs = 8 * heads
    return (pairs * 128 + 255) // 256 * 256 + pairs * 2 * 8192


def _mfma_bytes(B, H, T, D=128):
    """The three-kernel schedule: three map buffers per segment slot, at
    most three segments of at most ceil(T / n) frames held at once."""
    n = -(-T // 64)
    cap = -(-T // n)
    slot = (B * H * cap * D * D * 4 + 255) // 256 * 256
    return 3 * min(n, 3) * slot


SIZE_MAX = ctypes.c_size_t(-1).value
FRAME, FUSED, MFMA, PLAIN = 3, 2, 1, 0


def test_workspace_bytes():
    """With no device to ask, gdn_workspace_bytes gives the three-kernel
    schedule's size (an upper bound for the fused path's)."""
    L = F.lib()
    for s in (_shape(4, 16, 961, 880, 128), _shape(1, 16, 961, 880, 128), _shape(1, 3, 33, 40, 128)):
        assert L.gdn_workspace_bytes(ctypes.byref(s), BF16) == _mfma_bytes(s.B, s.H, s.T)
        assert L.gdn_workspace_bytes(ctypes.byref(s), BF16) >= \
            L.gdn_path_workspace_bytes(ctypes.byref(s), BF16, FUSED)
    # the 60 s workload: 16 segments of at most 61 frames, three held at once
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(1, 16, 961, 880, 128)), BF16) == 9 * 16 * 61 * 65536
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(T=0)), BF16) == 0
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(D=100)), BF16) == 0
    assert L.gdn_workspace_bytes(ctypes.byref(_shape()), 7) == 0
    s = _shape(1, 3, 5, 7, 48)
    assert L.gdn_workspace_bytes(ctypes.byref(s), F32) == 3 * ((15 * 48 * 48 * 4 + 255) // 256 * 256)
    assert L.gdn_workspace_bytes(None, BF16) == 0
    # a single frame: the split form's hand-off up to 16 heads, else none
    for B, H, S in ((1, 16, 880), (1, 1, 1), (4, 16, 5000), (1, 40, 64), (2, 8, 100), (1, 17, 880)):
        s = _shape(B, H, 1, S, 128)
        assert L.gdn_workspace_bytes(ctypes.byref(s), BF16) == _frame_bytes(H, S, B)
    assert _frame_bytes(16, 880) == 16 * 8 * (128 + 2 * 8192)
    assert _frame_bytes(17, 880) == 0 and _frame_bytes(8, 880, B=3) == 0
    prev = L.gdn_set_single_frame(0)
    try:
        s = _shape(1, 16, 1, 880, 128)
        assert L.gdn_workspace_bytes(ctypes.byref(s), BF16) == _mfma_bytes(1, 16, 1)
    finally:
        L.gdn_set_single_frame(prev)


def test_path_workspace_bytes():
    L = F.lib()
    pw = lambda s, path, dt=BF16: L.gdn_path_workspace_bytes(ctypes.byref(s), dt, path)
    # fused: rings for at most 16 heads at a time, independent of T and S
    f16 = pw(_shape(1, 16, 961, 880, 128), FUSED)
    assert 16 * 3 * 65536 <= f16 <= 80 << 20
    assert pw(_shape(4, 16, 961, 880, 128), FUSED) == f16
    assert pw(_shape(1, 16, 4000, 40, 128), FUSED) == f16
    f1, f2 = pw(_shape(1, 1, 961, 880, 128), FUSED), pw(_shape(1, 2, 961, 880, 128), FUSED)
    assert f16 - f1 == 15 * (f2 - f1)  # per-head rings
    # the three-kernel schedule: at most three segments of maps
    for B, H, T in ((1, 16, 961), (4, 16, 961), (1, 2, 64), (1, 2, 65), (1, 2, 200), (3, 5, 1)):
        assert pw(_shape(B, H, T, 880, 128), MFMA) == _mfma_bytes(B, H, T)
    # single frame: the split form's hand-off (none beyond 16 heads)
    assert pw(_shape(1, 16, 1, 880, 128), FRAME) == _frame_bytes(16, 880)
    for B, H, S in ((1, 1, 1), (1, 3, 64), (1, 3, 65), (2, 16, 1024), (1, 16, 1025), (1, 5, 5000)):
        assert pw(_shape(B, H, 1, S, 128), FRAME) == _frame_bytes(H, S, B)
    assert pw(_shape(1, 16, 2, 880, 128), FRAME) == SIZE_MAX
    assert pw(_shape(1, 16, 1, 880, 64), FRAME) == SIZE_MAX
    assert pw(_shape(1, 16, 1, 880, 128), FRAME, F32) == SIZE_MAX
    # the plain path: every frame's maps
    s = _shape(1, 3, 5, 7, 48)
    assert pw(s, PLAIN, F32) == 3 * ((15 * 48 * 48 * 4 + 255) // 256 * 256)
    # paths that cannot take the shape, and bad arguments
    assert pw(_shape(1, 16, 32, 880, 128), FUSED) == SIZE_MAX    # too short for the fused kernel
    assert pw(_shape(1, 16, 961, 880, 64), FUSED) == SIZE_MAX    # D != 128
    assert pw(_shape(1, 16, 961, 880, 128), FUSED, F32) == SIZE_MAX
    assert pw(_shape(1, 16, 961, 880, 128), MFMA, F32) == SIZE_MAX
    assert pw(_shape(1, 16, 961, 880, 128), 7) == SIZE_MAX
    assert pw(_shape(D=100), PLAIN) == SIZE_MAX
    assert L.gdn_path_workspace_bytes(None, BF16, FUSED) == SIZE_MAX
    assert pw(_shape(T=0), FUSED) == 0 and pw(_shape(S=0), MFMA) == 0


def test_noalloc_refuses_shapes_beyond_its_scratch_on_the_host():
    """Three-kernel calls too large for the built-in scratch are refused
    before any device is touched; invalid arguments are reported as by
    gdn_frame_fwd."""
    L = F.lib()

    def na(shape, **kw):
        a = dict(q=P[0], k=P[1], v=P[2], gamma=P[3], beta=P[4], state_in=None, out=P[5], state_out=P[6])
        a.update(kw)
        return L.gdn_frame_fwd_noalloc(ctypes.byref(shape) if shape else None, BF16, F32, a["q"], a["k"], a["v"],
                                       a["gamma"], a["beta"], a["state_in"], a["out"], a["state_out"], None)
    assert na(_shape(4, 16, 32, 16, 128)) == 10   # 3 x 2048 maps of 64 KiB: GDN_E_TOO_LARGE
    assert na(None) == NULLPTR
    assert na(_shape(D=100)) == UNSUP_D
    assert na(_shape(B=0), q=None, k=None, v=None, gamma=None, beta=None, out=None, state_out=None) == OK


def test_fused_status_rejects_null_workspace():
    assert F.lib().gdn_fused_status(None, None) == NULLPTR


# Fake, never-dereferenced device addresses, far apart.
P = [0x10_0000_0000 * (i + 1) for i in range(12)]


def fwd(shape, in_dt=BF16, out_dt=F32, q=P[0], k=P[1], v=P[2], gamma=P[3], beta=P[4],
        state_in=None, out=P[5], state_out=P[6], ws=P[7], wsb=None):
    L = F.lib()
    if wsb is None:
        wsb = L.gdn_workspace_bytes(ctypes.byref(shape), in_dt) if shape else 0
    return L.gdn_frame_fwd(ctypes.byref(shape) if shape else None, in_dt, out_dt, q, k, v, gamma,
                           beta, state_in, out, state_out, ws, wsb, None)


def test_frame_fwd_argument_errors():
    s = _shape()
    assert fwd(None) == NULLPTR
    for bad in ({"q": None}, {"k": None}, {"v": None}, {"gamma": None}, {"beta": None},
                {"out": None}, {"state_out": None}):
        assert fwd(s, **bad) == NULLPTR, bad
    assert fwd(_shape(B=-1)) == SHAPE
    assert fwd(_shape(T=-1)) == SHAPE
    assert fwd(_shape(S=-1)) == SHAPE
    assert fwd(_shape(D=100)) == UNSUP_D
    assert fwd(_shape(B=1 << 40, H=1 << 40)) == SHAPE
    assert fwd(_shape(B=1 << 12, H=1 << 12, T=2)) == SHAPE  # more frames than one launch can hold
    assert fwd(s, in_dt=5) == DTYPE
    assert fwd(s, out_dt=9) == DTYPE
    assert fwd(s, ws=None) == WORKSPACE
    assert fwd(s, wsb=1000) == WORKSPACE
    assert fwd(s, ws=P[7] + 8) == WORKSPACE  # misaligned


def test_key_scale_argument_errors():
    L = F.lib()
    s = _shape()
    wsb = L.gdn_workspace_bytes(ctypes.byref(s), BF16)

    def fks(ks, shape=s, k=P[1]):
        return L.gdn_frame_fwd_ks(ctypes.byref(shape), BF16, F32, P[0], k, P[2], P[3], P[4], None, ks,
                                  P[5], P[6], P[7], wsb, None)
    for bad in (float("nan"), float("inf"), -float("inf")):
        assert fks(bad) == VALUE
    assert fks(1.0, k=None) == NULLPTR     # other checks as gdn_frame_fwd's
    assert fks(1.0, shape=_shape(D=100)) == UNSUP_D
    bwsb = L.gdn_bwd_workspace_bytes(ctypes.byref(s), BF16)

    def bks(ks, dt=BF16):
        return L.gdn_frame_bwd_ks(ctypes.byref(s), dt, P[0], P[1], P[2], P[3], P[4], None, ks, P[5], None,
                                  P[6], P[7], P[8], P[9] + (1 << 30), P[9] + (2 << 30), P[11], P[10], bwsb,
                                  None)
    assert bks(float("nan")) == VALUE
    assert bks(float("inf")) == VALUE
    assert bks(1.0, dt=F32) == DTYPE


def test_empty_shapes_on_the_host():
    """Sizes of 0 are accepted by the whole-call entry points; a pointer may
    then be NULL exactly when its tensor is empty.  No heads: nothing to do
    (returns before touching a device).  The calls that set a state need a
    GPU and are tested there."""
    L = F.lib()
    none = dict(q=None, k=None, v=None, gamma=None, beta=None, out=None, state_out=None, ws=None, wsb=0)
    assert fwd(_shape(B=0), **none) == OK
    assert fwd(_shape(H=0, T=0, S=0), **none) == OK
    assert fwd(_shape(T=0), **none) == NULLPTR                   # state_out is needed
    assert fwd(_shape(S=0), **dict(none, state_out=P[6], beta=P[4])) == NULLPTR  # gamma is needed
    assert fwd(_shape(S=0), **dict(none, state_out=P[6], gamma=P[3])) == NULLPTR  # beta too
    assert fwd(_shape(T=0), **dict(none, state_out=P[6], state_in=P[6] + 4)) == ALIAS
    for s in (_shape(B=0), _shape(T=0), _shape(S=0), _shape(H=0, T=0)):
        assert L.gdn_workspace_bytes(ctypes.byref(s), BF16) == 0
        assert L.gdn_bwd_workspace_bytes(ctypes.byref(s), BF16) == 0
        assert L.gdn_path(ctypes.byref(s), BF16) == 0
    assert L.gdn_frame_fwd_ks(ctypes.byref(_shape(B=0)), BF16, F32, None, None, None, None, None, None, 0.5,
                              None, None, None, 0, None) == OK

    def bwd(shape, **kw):
        a = dict(q=None, k=None, v=None, gamma=None, beta=None, state=None, d_out=None, d_state_out=None,
                 dq=None, dk=None, dv=None, dgamma=None, dbeta=None, d_state_in=None)
        a.update(kw)
        return L.gdn_frame_bwd(ctypes.byref(shape), BF16, a["q"], a["k"], a["v"], a["gamma"], a["beta"],
                               a["state"], a["d_out"], a["d_state_out"], a["dq"], a["dk"], a["dv"], a["dgamma"],
                               a["dbeta"], a["d_state_in"], None, 0, None)
    assert bwd(_shape(B=0)) == OK
    assert bwd(_shape(T=0)) == NULLPTR                                      # d_state_in is needed
    assert bwd(_shape(S=0), gamma=P[3], beta=P[4], d_state_in=P[11], dbeta=P[9]) == NULLPTR   # dgamma
    assert bwd(_shape(S=0, D=64)) == UNSUP_D                               # the backward is D = 128 only
    assert L.gdn_build_maps(ctypes.byref(_shape(T=0)), BF16, P[0], P[1], P[2], P[3], None) == SHAPE
    assert L.gdn_state_pass(ctypes.byref(_shape(H=0)), P[0], P[1], P[2], P[3], None, P[4], P[5], None) == SHAPE


def test_frame_fwd_alias_errors():
    s = _shape()
    assert fwd(s, out=P[0]) == ALIAS                 # out over q
    assert fwd(s, state_out=P[5] + 64) == ALIAS      # state_out inside out
    assert fwd(s, state_in=P[6] + 4) == ALIAS        # partial overlap with state_out
    assert fwd(s, ws=P[1]) == ALIAS                  # workspace over k
    assert fwd(s, gamma=P[6]) == ALIAS               # state_out over gamma


def test_timed_needs_output_array():
    L = F.lib()
    s = _shape()
    wsb = L.gdn_workspace_bytes(ctypes.byref(s), BF16)
    ms, nl = (ctypes.c_float * 3)(), (ctypes.c_int * 3)()
    assert L.gdn_frame_fwd_timed(ctypes.byref(s), BF16, F32, P[0], P[1], P[2], P[3], P[4], None, P[5],
                                 P[6], P[7], wsb, None, None, nl) == NULLPTR
    assert L.gdn_frame_fwd_timed(ctypes.byref(s), BF16, F32, P[0], P[1], P[2], P[3], P[4], None, P[5],
                                 P[6], P[7], wsb, None, ms, None) == NULLPTR


def test_backward_argument_errors():
    L = F.lib()
    s = _shape()
    wsb = L.gdn_bwd_workspace_bytes(ctypes.byref(s), BF16)
    per = 2 * 3 * 128 * 128 * 4
    partials = 6 * 8 * 2 * 4  # frames x 8 parts x (dgamma, dbeta) floats
    assert wsb == 5 * ((per + 255) // 256 * 256) + (partials + 255) // 256 * 256 + 2 * 128 * 128 * 4

    def bwd(shape=s, dt=BF16, d_state_out=None, d_state_in=P[11], ws=P[10], wsb=wsb, **kw):
        a = dict(q=P[0], k=P[1], v=P[2], gamma=P[3], beta=P[4], state=None, d_out=P[5], dq=P[6], dk=P[7],
                 dv=P[8], dgamma=P[9] + (1 << 30), dbeta=P[9] + (2 << 30))
        a.update(kw)
        return L.gdn_frame_bwd(ctypes.byref(shape) if shape else None, dt, a["q"], a["k"], a["v"], a["gamma"],
                               a["beta"], a["state"], a["d_out"], d_state_out, a["dq"], a["dk"], a["dv"],
                               a["dgamma"], a["dbeta"], d_state_in, ws, wsb, None)
    assert bwd(shape=None) == NULLPTR
    assert bwd(dt=F32) == DTYPE
    assert bwd(shape=_shape(D=64), wsb=L.gdn_bwd_workspace_bytes(ctypes.byref(_shape(D=64)), BF16)) == UNSUP_D
    assert bwd(d_out=None) == NULLPTR
    assert bwd(d_state_in=None) == NULLPTR
    assert bwd(wsb=wsb - 1) == WORKSPACE
    assert bwd(dq=P[0]) == ALIAS                       # a gradient over q
    assert bwd(dk=P[6]) == ALIAS                       # two gradients in one buffer
    assert bwd(d_state_out=P[11] + 4) == ALIAS         # partial overlap of the state gradients


def test_stage_argument_errors():
    L = F.lib()
    s = _shape()
    assert L.gdn_build_maps(ctypes.byref(s), BF16, None, P[1], P[2], P[3], None) == NULLPTR
    assert L.gdn_build_maps(ctypes.byref(s), 3, P[0], P[1], P[2], P[3], None) == DTYPE
    assert L.gdn_build_maps(ctypes.byref(s), BF16, P[0], P[1], P[0], P[3], None) == ALIAS
    assert L.gdn_build_maps(ctypes.byref(s), BF16, P[0], P[1], P[2], P[2] + 4, None) == ALIAS
    assert L.gdn_state_pass(ctypes.byref(s), P[0], P[1], P[2], P[3], None, P[4], None, None) == NULLPTR
    assert L.gdn_state_pass(ctypes.byref(_shape(D=48 + 1)), P[0], P[1], P[2], P[3], None, P[4], P[5],
                            None) == UNSUP_D
    assert L.gdn_state_pass(ctypes.byref(s), P[0], P[1], P[2], P[3], None, P[0], P[5], None) == ALIAS
    assert L.gdn_output(ctypes.byref(s), BF16, F32, P[0], P[1], P[1], None) == ALIAS
    assert L.gdn_output(ctypes.byref(s), BF16, 4, P[0], P[1], P[2], None) == DTYPE
    assert L.gdn_output(ctypes.byref(_shape(S=0)), BF16, F32, P[0], P[1], P[2], None) == SHAPE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from frame_wise_gated_fwd_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_attention_argument_errors_on_the_host():
    """gdn_attn_fwd rejects bad arguments before launching anything."""
    from frame_wise_gated_fwd_amd._lib import AttnLayout
    L = F.lib()

    def att(shape=None, dt=BF16, lay=(1, 1, 4, 2), q=P[0], k=P[1], v=P[2], out=P[3], lse=P[4]):
        s = shape if shape is not None else _shape(1, 2, 9, 40, 128)
        lo = AttnLayout(*lay) if lay is not None else None
        return L.gdn_attn_fwd(ctypes.byref(s), dt, ctypes.byref(lo) if lo is not None else None, q, k, v, out, lse,
                              None)
    assert L.gdn_attn_fwd(None, BF16, None, P[0], P[1], P[2], P[3], None, None) == NULLPTR
    assert att(lay=None) == NULLPTR
    for bad in ({"q": None}, {"k": None}, {"v": None}, {"out": None}):
        assert att(**bad) == NULLPTR, bad
    assert att(dt=F32) == DTYPE
    assert att(dt=7) == DTYPE
    assert att(shape=_shape(1, 2, 9, 40, 64)) == UNSUP_D
    assert att(shape=_shape(1, -2, 9, 40, 128)) == SHAPE
    assert att(shape=_shape(1, 1, 1 << 16, 1 << 14, 128)) == SHAPE   # 2^30 tokens per head
    for lay in ((-1, 1, 4, 2), (1, 0, 4, 2), (1, 1, 0, 2), (1, 1, 4, 0)):
        assert att(lay=lay) == VALUE, lay
    assert att(out=P[0]) == ALIAS                 # out over q
    assert att(lse=P[3] + 64) == ALIAS            # lse inside out
    assert att(shape=_shape(0, 2, 9, 40, 128), q=None, k=None, v=None, out=None, lse=None) == OK


def test_gated_argument_errors_on_the_host():
    L = F.lib()
    s = _shape()
    wsb = L.gdn_workspace_bytes(ctypes.byref(s), BF16)

    def gated(shape=s, ga=P[7] + (1 << 33), gb=P[7] + (2 << 33), A=P[8], bias=P[8] + 4096, gam=P[9], bet=P[10],
              ks=1.0, ws=P[11], wsb_=wsb):
        return L.gdn_frame_fwd_gated(ctypes.byref(shape), BF16, F32, P[0], P[1], P[2], ga, gb, A, bias, None, ks,
                                     P[5], P[6], gam, bet, ws, wsb_, None)
    for bad in ({"ga": None}, {"gb": None}, {"A": None}, {"bias": None}, {"gam": None}, {"bet": None}):
        assert gated(**bad) == NULLPTR, bad
    assert gated(ks=float("nan")) == VALUE
    assert gated(shape=_shape(S=0), ws=None, wsb_=0) == SHAPE      # a frame's gates average its tokens
    assert gated(gam=P[5]) == ALIAS                               # gamma written over out
    assert gated(gam=P[9], bet=P[9] + 8) == ALIAS                 # gamma and beta overlap
    assert gated(ga=P[5]) == ALIAS                                # out written over a gate input
    assert gated(shape=_shape(B=0), ws=None, wsb_=0) == OK


def test_single_frame_workspace_is_optional_but_checked():
    """A single-frame call (bf16, D = 128, T = 1) needs no workspace: without
    one, or with one too small or misaligned for the two-workgroup form, the
    host checks pass and the call goes on to the device (here, with no GPU,
    to GDN_E_HIP).  A workspace big enough for that form is checked like any
    other: overlapping an input or output is GDN_E_ALIAS."""
    L = F.lib()
    prev = L.gdn_set_single_frame(1)
    try:
        s = _shape(1, 16, 1, 880, 128)
        need = L.gdn_workspace_bytes(ctypes.byref(s), BF16)
        assert need == _frame_bytes(16, 880)
        for ws, wsb in ((None, 0), (P[7], need - 1), (P[7] + 8, need), (P[7], need)):
            assert fwd(s, ws=ws, wsb=wsb) == HIP, (ws, wsb)
        assert fwd(s, ws=P[1], wsb=need) == ALIAS        # over k
        assert fwd(s, ws=P[6] - 256, wsb=need) == ALIAS  # over state_out
        assert fwd(s, ws=P[1], wsb=need - 1) == HIP      # too small to be used: not checked
    finally:
        L.gdn_set_single_frame(prev)
