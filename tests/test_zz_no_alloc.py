"""gdn_frame_fwd_noalloc (the entry point for callers that cannot allocate)
against gdn_frame_fwd through the C ABI: two calls in a row on one GPU, the
second with a smaller input (so it runs on what the first left in the shared
scratch array), a third on the three-kernel path and a fourth on the
single-frame kernels (two head groups).  Both entry points run
the same kernels, so the results must agree bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import frame_wise_gated_fwd_amd as F
from frame_wise_gated_fwd_amd._lib import Shape, GDN_BF16, GDN_F32
from synth import Workload

from gpu_util import device_inputs, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOO_LARGE = 10


def _noalloc(x, w, out_dtype=torch.float32):
    L = F.lib()
    shp = Shape(w.B, w.H, w.T, w.S, w.D)
    out = torch.full((w.B, w.H, w.T, w.S, w.D), float("nan"), dtype=out_dtype, device=DEV)
    st = torch.full((w.B, w.H, w.D, w.D), float("nan"), dtype=torch.float32, device=DEV)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.gdn_frame_fwd_noalloc(ctypes.byref(shp), GDN_BF16, GDN_BF16 if out_dtype == torch.bfloat16 else GDN_F32,
                                 P(x["q"]), P(x["k"]), P(x["v"]), P(x["gamma"]), P(x["beta"]), P(x["state"]),
                                 P(out), P(st), stream)
    return rc, out, st


@pytest.mark.parametrize("w", [
    Workload(name="noalloc_big", B=1, H=16, T=100, S=200, D=128, in_dtype="bf16", seed=71,
             gamma_range=(0.95, 1.0), beta_kind="sigmoid_normal", state_std=0.02),
], ids=lambda w: w.name)
def test_noalloc_matches_frame_fwd_on_successive_calls(w):
    smaller = w.with_(name="noalloc_small", H=5, T=40, S=64, seed=72)
    short = w.with_(name="noalloc_three_kernel", H=3, T=8, S=50, seed=73, state_std=None)
    single = w.with_(name="noalloc_single_frame", H=20, T=1, S=880, seed=75)
    for wk, odt in ((w, torch.float32), (smaller, torch.bfloat16), (short, torch.float32),
                    (single, torch.float32)):
        log(f"noalloc {wk.name}: B={wk.B} H={wk.H} T={wk.T} S={wk.S} out {odt}")
        x = device_inputs(wk, DEV)
        ref_out, ref_st = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"], out_dtype=odt)
        rc, out, st = _noalloc(x, wk, odt)
        torch.cuda.synchronize()
        assert rc == 0, rc
        assert torch.equal(out, ref_out), wk.name
        assert torch.equal(st, ref_st), wk.name


def test_noalloc_rejects_a_call_beyond_its_scratch():
    """16 x 4 heads of 32 frames take the three-kernel path, whose maps
    (3 x 2048 x 64 KiB) exceed the scratch array: refused before any launch."""
    w = Workload(name="noalloc_too_large", B=4, H=16, T=32, S=16, D=128, in_dtype="bf16", seed=74,
                 gamma_range=(0.95, 1.0), beta_kind="sigmoid_normal", state_std=None)
    L = F.lib()
    assert L.gdn_workspace_bytes(ctypes.byref(Shape(w.B, w.H, w.T, w.S, w.D)), GDN_BF16) > 96 << 20
    x = device_inputs(w, DEV)
    rc, out, st = _noalloc(x, w)
    torch.cuda.synchronize()
    assert rc == TOO_LARGE
    assert bool(torch.isnan(st).all())  # nothing was written
