"""Property test of gdn_frame_fwd's argument checks on the host (no GPU):
random shapes, dtypes, key scales, pointers and workspaces against a model
of the contract written from include/gdn.h.  Only calls the model says
return before any launch are made (errors, and shapes with no heads)."""
import ctypes
import math

import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import frame_wise_gated_fwd_amd as F
from frame_wise_gated_fwd_amd._lib import Shape

OK, NULLPTR, SHAPE, DTYPE, UNSUP_D, WORKSPACE, ALIAS, HIP, VALUE = range(9)
MAX_FRAMES = (1 << 24) - 1
I64 = (1 << 63) - 1
BASE = 0x40_0000_0000


def _mul(a, b):
    r = a * b
    return r if r <= I64 else None


def model(shape, in_dt, out_dt, ks, ptrs, ws, wsb):
    """(status, launches) per the contract: the checks in the order the
    header states them (shape, key scale, dtypes, pointers, workspace of the
    planned path, aliasing)."""
    if shape is None:
        return NULLPTR, False
    B, H, T, S, D = shape
    if min(B, H, T, S) < 0 or D < 1:
        return SHAPE, False
    if not (16 <= D <= 128 and D % 16 == 0):
        return UNSUP_D, False
    if S > (2**31 - 1) // 256:
        return SHAPE, False
    heads = _mul(B, H)
    if heads is None or heads > MAX_FRAMES:
        return SHAPE, False
    frames = _mul(heads, T)
    if frames is None or frames > MAX_FRAMES:
        return SHAPE, False
    t = _mul(frames, S)
    in_elems = None if t is None else _mul(t, D)
    map_elems = _mul(frames, D * D)
    if in_elems is None or map_elems is None or in_elems > 1 << 56 or map_elems > 1 << 56:
        return SHAPE, False
    if not math.isfinite(ks):
        return VALUE, False
    if in_dt not in (0, 1) or out_dt not in (0, 1):
        return DTYPE, False
    need_in, need_fr, need_st = in_elems > 0, frames > 0, heads > 0
    q, k, v, gamma, beta, state_in, out, state_out = ptrs
    if (need_in and None in (q, k, v, out)) or (need_fr and None in (gamma, beta)) or (need_st and state_out is None):
        return NULLPTR, False
    need = 0 if in_elems == 0 else _planned_need(shape, in_dt, frames, map_elems)
    if need > 0 and (ws is None or wsb < need or ws % 256):
        return WORKSPACE, False
    isz, osz = (2 if in_dt == 1 else 4), (2 if out_dt == 1 else 4)
    stb, gb = heads * D * D * 4, frames * 4
    outs = [(out, in_elems * osz), (state_out, stb), (ws, need)]
    ins = [(q, in_elems * isz), (k, in_elems * isz), (v, in_elems * isz), (gamma, gb), (beta, gb),
           (state_in, stb if state_in is not None else 0)]

    def overlap(a, b):
        return a[0] is not None and b[0] is not None and a[1] and b[1] and a[0] < b[0] + b[1] and b[0] < a[0] + a[1]
    for i, o in enumerate(outs):
        for j in ins:
            if overlap(o, j) and not (o[0] == j[0] and o[1] == j[1] and o[0] == state_out and j[0] == state_in):
                return ALIAS, False
        for o2 in outs[i + 1:]:
            if overlap(o, o2):
                return ALIAS, False
    return OK, need_st


def _planned_need(shape, in_dt, frames, map_elems):
    """Workspace of the path the call plans before asking the device: the
    fused kernel's (bf16, D = 128, T > 32, as gdn_path_workspace_bytes
    reports it), the three-kernel schedule's three segments of maps (bf16,
    D = 128; none for a single frame), else every frame's maps."""
    B, H, T, S, D = shape
    if in_dt == 1 and D == 128 and T > 32:
        return F.lib().gdn_path_workspace_bytes(ctypes.byref(Shape(*shape)), in_dt, 2)
    if in_dt == 1 and D == 128:
        n = -(-T // 64)
        cap = -(-T // n)
        mfma = 3 * min(n, 3) * ((B * H * cap * D * D * 4 + 255) // 256 * 256)
        return 0 if T == 1 else mfma  # a single frame needs no workspace
    return 3 * ((map_elems * 4 + 255) // 256 * 256)


sizes = st.one_of(st.integers(0, 3), st.sampled_from([-1, 5, 64, 65, 880, 1 << 20, 1 << 40]))
dims = st.sampled_from([0, 8, 16, 48, 100, 128, 128, 144])


def _ptr(slot, off):
    # slot 0: NULL; else one of 12 addresses far apart, at times plus a small
    # offset (a partial overlap with whatever else uses the slot)
    return None if slot == 0 else BASE * slot + off


ptr = st.builds(_ptr, st.integers(0, 12), st.sampled_from([0, 0, 0, 0, 4, 256]))


@settings(max_examples=600, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(shape=st.one_of(st.none(), st.tuples(sizes, sizes, sizes, sizes, dims)),
       in_dt=st.sampled_from([0, 1, 1, 1, 2]), out_dt=st.sampled_from([0, 0, 0, 1, -1]),
       ks=st.sampled_from([1.0, 1.0, 1.0, 0.5, math.nan, math.inf]), ptrs=st.lists(ptr, min_size=8, max_size=8),
       ws=ptr, wsb=st.sampled_from([0, 1 << 10, 1 << 30, 1 << 45]))
def test_frame_fwd_argument_checks_match_the_contract(shape, in_dt, out_dt, ks, ptrs, ws, wsb):
    want, launches = model(shape, in_dt, out_dt, ks, ptrs, ws, wsb)
    if launches:
        return  # a valid call that would run kernels: GPU tests cover those
    L = F.lib()
    shp = None if shape is None else Shape(*shape)
    q, k, v, gamma, beta, state_in, out, state_out = ptrs
    got = L.gdn_frame_fwd_ks(ctypes.byref(shp) if shp else None, in_dt, out_dt, q, k, v, gamma, beta, state_in, ks,
                             out, state_out, ws, wsb, None)
    assert got == want, (shape, in_dt, out_dt, ks, ptrs, ws, wsb, got, want)
