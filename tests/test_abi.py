"""The C ABI on the host, with no GPU: the library loads, exports every symbol
include/gdn.h declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

import frame_wise_gated_fwd_amd as F
from frame_wise_gated_fwd_amd._lib import SIGNATURES, Shape

HEADER = os.path.join(os.path.dirname(__file__), "..", "include", "gdn.h")

OK, NULLPTR, SHAPE, DTYPE, UNSUP_D, WORKSPACE, ALIAS, HIP, VALUE = range(9)
F32, BF16 = 0, 1


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", txt)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(SIGNATURES)


def test_library_exports_every_declared_symbol():
    L = F.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.gdn_abi_version() == 2


def test_status_strings():
    L = F.lib()
    for s in range(9):
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


def test_workspace_bytes():
    L = F.lib()
    for s in (_shape(4, 16, 961, 880, 128), _shape(1, 16, 961, 880, 128)):
        per = s.B * s.H * s.T * 128 * 128 * 4
        assert L.gdn_workspace_bytes(ctypes.byref(s), BF16) == 3 * ((per + 255) // 256 * 256)
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(T=0)), BF16) == 0
    assert L.gdn_workspace_bytes(ctypes.byref(_shape(D=100)), BF16) == 0
    assert L.gdn_workspace_bytes(ctypes.byref(_shape()), 7) == 0
    s = _shape(1, 3, 5, 7, 48)
    assert L.gdn_workspace_bytes(ctypes.byref(s), F32) == 3 * ((15 * 48 * 48 * 4 + 255) // 256 * 256)
    assert L.gdn_workspace_bytes(None, BF16) == 0


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
