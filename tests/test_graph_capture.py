"""The forward captured into a HIP graph and replayed: every replay, on fresh
inputs written into the captured buffers, must equal an eager call on the
same buffers bit for bit.

Covered: the fused kernel through gdn_frame_fwd_noalloc (the entry point
meant for capture) and through gdn_frame_fwd, over more than 16 heads (two
launches of it, each after its flag-reset kernel), the single-frame kernel
in both of its forms, and the overlapped
three-kernel schedule, whose builds, state passes and outputs fork onto the
library's own streams and join back.  Each capture follows an eager call of
the same shape, since the first call on a device queries it (a probe kernel
on the null stream, which a capture may not contain).  Between replays the
program does eager work of its own and synchronises."""
import ctypes

import pytest
import torch

import frame_wise_gated_fwd_amd as F
from frame_wise_gated_fwd_amd._lib import Shape, GDN_BF16, GDN_F32
from synth import Workload

from gpu_util import device_inputs, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3

BASE = Workload(name="graph", B=1, H=20, T=40, S=64, D=128, in_dtype="bf16", seed=91,
                gamma_range=(0.95, 1.0), beta_kind="sigmoid_normal", state_std=0.02)


def _input_sets(w, n):
    return [device_inputs(w.with_(seed=w.seed + 10 * i), DEV) for i in range(n)]


def _load(static, x):
    for key, t in static.items():
        if t is not None:
            t.copy_(x[key])


def _eager(static, odt):
    return F.frame_fwd(static["q"], static["k"], static["v"], static["gamma"], static["beta"], static["state"],
                       out_dtype=odt)


def _capture(fn):
    """fn run once eagerly on a side stream, then captured."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    torch.cuda.synchronize()
    return g, res


def _replay_and_check(g, static, sets, out, st, odt, name):
    other = torch.randn(1024, 1024, device=DEV)
    for i, x in enumerate(sets):
        _load(static, x)
        out.fill_(float("nan"))
        st.fill_(float("nan"))
        torch.cuda.synchronize()
        log(f"{name}: replay {i}")
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_st = _eager(static, odt)
        other = other @ other.T / 1024.0  # the program's own work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"{name}: replay {i} out"
        assert torch.equal(st, ref_st), f"{name}: replay {i} state"
    assert torch.isfinite(other).all()


@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16], ids=["f32_out", "bf16_out"])
def test_noalloc_fused_in_a_graph(odt):
    w = BASE
    L = F.lib()
    shp = Shape(w.B, w.H, w.T, w.S, w.D)
    assert L.gdn_path(ctypes.byref(shp), GDN_BF16) == 2, "shape must take the fused kernel"
    sets = _input_sets(w, REPLAYS + 1)
    static = {key: t.clone() for key, t in sets[0].items()}
    out = torch.empty((w.B, w.H, w.T, w.S, w.D), dtype=odt, device=DEV)
    st = torch.empty((w.B, w.H, w.D, w.D), dtype=torch.float32, device=DEV)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())

    def call():
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = L.gdn_frame_fwd_noalloc(ctypes.byref(shp), GDN_BF16, GDN_BF16 if odt == torch.bfloat16 else GDN_F32,
                                     P(static["q"]), P(static["k"]), P(static["v"]), P(static["gamma"]),
                                     P(static["beta"]), P(static["state"]), P(out), P(st), stream)
        assert rc == 0, rc

    log(f"noalloc fused graph: H={w.H} T={w.T} S={w.S} out {odt}")
    g, _ = _capture(call)
    _replay_and_check(g, static, sets[1:], out, st, odt, "noalloc fused graph")


def test_frame_fwd_fused_in_a_graph():
    w = BASE.with_(H=5, seed=93)
    sets = _input_sets(w, REPLAYS + 1)
    static = {key: t.clone() for key, t in sets[0].items()}
    log(f"frame_fwd fused graph: H={w.H} T={w.T} S={w.S}")
    g, (out, st) = _capture(lambda: _eager(static, torch.float32))
    _replay_and_check(g, static, sets[1:], out, st, torch.float32, "frame_fwd fused graph")


@pytest.mark.parametrize("H", [20, 16])
def test_single_frame_kernels_in_a_graph(H):
    """The single-frame kernel: 20 heads take one workgroup per 16-row block;
    16 heads two, which swap partial sums through per-block words that every
    call (eager or replayed) leaves ready for the next."""
    w = BASE.with_(H=H, T=1, S=880, seed=97)
    assert F.lib().gdn_path(ctypes.byref(Shape(w.B, w.H, w.T, w.S, w.D)), GDN_BF16) == 3
    sets = _input_sets(w, REPLAYS + 1)
    static = {key: t.clone() for key, t in sets[0].items()}
    log(f"single-frame graph: H={w.H} S={w.S}")
    g, (out, st) = _capture(lambda: _eager(static, torch.float32))
    _replay_and_check(g, static, sets[1:], out, st, torch.float32, "single-frame graph")


def test_overlapped_three_kernel_schedule_in_a_graph():
    """T = 100 frames in two segments of at most 64: builds on the caller's
    stream, state passes and outputs on the library's two side streams."""
    w = BASE.with_(H=3, T=100, S=50, seed=95)
    prev = F.set_fused(False)
    try:
        L = F.lib()
        assert L.gdn_path(ctypes.byref(Shape(w.B, w.H, w.T, w.S, w.D)), GDN_BF16) == 1
        sets = _input_sets(w, REPLAYS + 1)
        static = {key: t.clone() for key, t in sets[0].items()}
        log(f"three-kernel graph: H={w.H} T={w.T} S={w.S}")
        g, (out, st) = _capture(lambda: _eager(static, torch.float32))
        _replay_and_check(g, static, sets[1:], out, st, torch.float32, "three-kernel graph")
    finally:
        F.set_fused(prev)
