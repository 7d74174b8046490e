"""ctypes loader for libgdn.so (the C ABI declared in include/gdn.h and
include/gdn_attn.h).

The library is built in-tree by frame_wise_gated_fwd_amd.build.  Loading
fails loudly when it is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GDN_LIB", os.path.join(_PKG, "libgdn.so"))

GDN_OK = 0
GDN_F32 = 0
GDN_BF16 = 1
GDN_PATH_PLAIN, GDN_PATH_MFMA, GDN_PATH_FUSED, GDN_PATH_FRAME = 0, 1, 2, 3

STATUS_NAMES = {0: "GDN_OK", 1: "GDN_E_NULLPTR", 2: "GDN_E_SHAPE", 3: "GDN_E_DTYPE",
                4: "GDN_E_UNSUPPORTED_D", 5: "GDN_E_WORKSPACE", 6: "GDN_E_ALIAS", 7: "GDN_E_HIP",
                8: "GDN_E_VALUE", 9: "GDN_E_TIMEOUT", 10: "GDN_E_TOO_LARGE"}

# Every symbol include/gdn.h declares, with (restype, argtypes).
_vp, _cvp = ctypes.c_void_p, ctypes.c_void_p
_sz, _i, _f = ctypes.c_size_t, ctypes.c_int, ctypes.c_float


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64),
                ("S", ctypes.c_int64), ("D", ctypes.c_int64)]


_PS = ctypes.POINTER(Shape)


class AttnLayout(ctypes.Structure):
    """gdn_attn_layout (include/gdn_attn.h)."""
    _fields_ = [("sink", ctypes.c_int64), ("first_chunk", ctypes.c_int64), ("chunk", ctypes.c_int64),
                ("window", ctypes.c_int64)]

SIGNATURES = {
    "gdn_abi_version": (_i, []),
    "gdn_status_str": (ctypes.c_char_p, [_i]),
    "gdn_supports_d": (_i, [ctypes.c_int64]),
    "gdn_path": (_i, [_PS, _i]),
    "gdn_set_fused": (_i, [_i]),
    "gdn_set_single_frame": (_i, [_i]),
    "gdn_workspace_bytes": (_sz, [_PS, _i]),
    "gdn_path_workspace_bytes": (_sz, [_PS, _i, _i]),
    "gdn_fused_status": (_i, [_cvp, _vp]),
    "gdn_set_spin_limit": (ctypes.c_uint, [ctypes.c_uint]),
    "gdn_frame_fwd": (_i, [_PS, _i, _i, _cvp, _cvp, _cvp, _cvp, _cvp, _cvp, _vp, _vp, _vp, _sz, _vp]),
    "gdn_frame_fwd_noalloc": (_i, [_PS, _i, _i, _cvp, _cvp, _cvp, _cvp, _cvp, _cvp, _vp, _vp, _vp]),
    "gdn_frame_fwd_gated": (_i, [_PS, _i, _i, _cvp, _cvp, _cvp, _cvp, _cvp, _cvp, _cvp, _cvp, _f, _vp, _vp, _vp,
                                 _vp, _vp, _sz, _vp]),
    "gdn_frame_fwd_ks": (_i, [_PS, _i, _i, _cvp, _cvp, _cvp, _cvp, _cvp, _cvp, _f, _vp, _vp, _vp, _sz, _vp]),
    "gdn_frame_fwd_timed": (_i, [_PS, _i, _i, _cvp, _cvp, _cvp, _cvp, _cvp, _cvp, _vp, _vp, _vp, _sz, _vp,
                                 ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int)]),
    "gdn_bwd_workspace_bytes": (_sz, [_PS, _i]),
    "gdn_frame_bwd": (_i, [_PS, _i, _cvp, _cvp, _cvp, _cvp, _cvp, _cvp, _cvp, _cvp, _vp, _vp, _vp, _vp, _vp,
                           _vp, _vp, _sz, _vp]),
    "gdn_frame_bwd_ks": (_i, [_PS, _i, _cvp, _cvp, _cvp, _cvp, _cvp, _cvp, _f, _cvp, _cvp, _vp, _vp, _vp, _vp,
                              _vp, _vp, _vp, _sz, _vp]),
    "gdn_attn_fwd": (_i, [_PS, _i, ctypes.POINTER(AttnLayout), _cvp, _cvp, _cvp, _vp, _vp, _vp]),
    "gdn_build_maps": (_i, [_PS, _i, _cvp, _cvp, _vp, _vp, _vp]),
    "gdn_state_pass": (_i, [_PS, _cvp, _cvp, _cvp, _cvp, _cvp, _vp, _vp, _vp]),
    "gdn_output": (_i, [_PS, _i, _i, _cvp, _cvp, _vp, _vp]),
}

_lib = None


class GDNError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS_NAMES.get(status, str(status))
        msg = lib().gdn_status_str(status).decode() if _lib is not None else ""
        super().__init__(f"{where}: {name} ({msg})")


def lib():
    """The loaded library (loads it on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m frame_wise_gated_fwd_amd.build` "
                "(the GDN forward has no non-HIP implementation)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status: int, where: str) -> None:
    if status != GDN_OK:
        raise GDNError(status, where)
