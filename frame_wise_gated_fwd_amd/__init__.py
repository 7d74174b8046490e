"""Frame-wise Gated DeltaNet forward on AMD Instinct MI355X (gfx950).

The computation lives in libgdn.so (HIP kernels behind the C ABI in
include/gdn.h and include/gdn_attn.h); this package only marshals torch
tensors into it.
"""
from .api import (frame_fwd, frame_bwd, build_maps, state_pass, output, workspace_bytes, set_fused, set_single_frame, attn_fwd,
                  frame_fwd_gated)
from ._lib import lib, GDNError, LIB_PATH

__all__ = ["frame_fwd", "frame_bwd", "build_maps", "state_pass", "output", "workspace_bytes", "set_fused", "set_single_frame",
           "attn_fwd", "frame_fwd_gated", "lib", "GDNError", "LIB_PATH"]
