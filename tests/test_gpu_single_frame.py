"""The single-frame kernels (T == 1, bf16, D == 128: the call of frame-by-frame
generation) through the C ABI: against the fp64 oracle at float32-grade
tolerance (relative L2 <= 1e-5 for the output and the state, every head and
frame on its own), against the three-kernel path (the same step with the
frame's tokens summed in another order), over many calls in a row, and on
their edge cases: head counts that are not a multiple of 8, one
token, more token tiles than waves, a zero state, the state updated in
place, bf16 output, the key scale and gates from activations."""
import ctypes

import pytest
import torch

import frame_wise_gated_fwd_amd as F
from frame_wise_gated_fwd_amd._lib import Shape, GDN_BF16, GDN_PATH_FRAME, GDN_PATH_MFMA
from synth import CLIP_5S, Workload

from gpu_util import device_inputs, rel_l2, log
from test_gpu_parity import _forward_parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-5


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _path(w):
    return F.lib().gdn_path(ctypes.byref(Shape(w.B, w.H, w.T, w.S, w.D)), GDN_BF16)


def _both_paths(fn):
    """fn() with the single-frame kernels, then through the three-kernel path."""
    a = fn()
    prev = F.set_single_frame(False)
    try:
        b = fn()
    finally:
        F.set_single_frame(prev)
    torch.cuda.synchronize()
    return a, b


def _rel(a, b):
    return rel_l2(a.double().cpu().numpy(), b.double().cpu().numpy())


@pytest.mark.parametrize("B,H,S,state", [
    (1, 16, 880, True),    # one 720p latent frame of 16 heads: 14 token tiles per head
    (1, 16, 880, False),   # zero state (no state_in)
    (1, 3, 100, True),     # 3 heads (the rows launch rounds up to 8); a ragged tile (64 + 36 tokens)
    (1, 20, 200, True),    # 20 heads: 24 heads' worth of row workgroups, 4 idle
    (2, 8, 1, True),       # one token: seven waves of each row workgroup without a tile
    (1, 9, 17, True),      # 17 tokens, 9 heads
    (1, 4, 3000, True),    # 47 tiles: 5 or 6 per wave of a row workgroup, 16 outputs of 3 tiles (the last 2)
], ids=lambda v: str(v))
def test_single_frame_matches_oracle(B, H, S, state):
    w = Workload(name=f"frame1_{B}_{H}_{S}", B=B, H=H, T=1, S=S, D=128, in_dtype="bf16", seed=300 + H + S,
                 gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal", state_std=0.05 if state else None, tol=TOL)
    assert _path(w) == GDN_PATH_FRAME
    _forward_parity(w)


def test_single_frame_calls_match_oracle_over_many_frames():
    """16 heads of 880 tokens, 24 frames one call each, the state updated in
    place: every frame and the final state against the oracle."""
    w = CLIP_5S.with_(T=24, name="frame1_stream24", state_std=0.02, tol=TOL)
    x = device_inputs(w, DEV)
    state = x["state"].clone()
    out = torch.empty(x["q"].shape, dtype=torch.float32, device=DEV)
    for t in range(w.T):
        sl = slice(t, t + 1)
        o, _ = F.frame_fwd(x["q"][:, :, sl].contiguous(), x["k"][:, :, sl].contiguous(),
                           x["v"][:, :, sl].contiguous(), x["gamma"][:, :, sl].contiguous(),
                           x["beta"][:, :, sl].contiguous(), state, state_out=state)
        out[:, :, sl] = o
    torch.cuda.synchronize()
    from gpu_util import oracle_heads, RelL2
    ro, rs = RelL2(), RelL2()
    worst = 0.0
    for b, h, O, M in oracle_heads(w, [(0, h) for h in range(w.H)], None):
        og = out[b, h].double().cpu().numpy()
        ro.add(og, O)
        rs.add(state[b, h].double().cpu().numpy(), M)
        worst = max(worst, max(rel_l2(og[i], O[i]) for i in range(w.T)))
    log(f"  24 single-frame calls: relL2 O={ro.value:.3e} state={rs.value:.3e}, worst frame {worst:.3e}")
    assert ro.value <= TOL and rs.value <= TOL and worst <= TOL


def test_single_frame_agrees_with_three_kernel_path():
    """Both paths compute the same step; only the order in which a frame's
    880 tokens are summed differs."""
    w = CLIP_5S.with_(T=1, name="frame1_vs_mfma", state_std=0.02)
    x = device_inputs(w, DEV)
    (o1, s1), (o2, s2) = _both_paths(
        lambda: F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"]))
    ro, rs = _rel(o1, o2), _rel(s1, s2)
    log(f"  single-frame vs three-kernel: relL2 O={ro:.3e} state={rs:.3e}")
    assert ro <= 4e-6 and rs <= 1e-6


def test_single_frame_deterministic_and_in_place():
    w = CLIP_5S.with_(T=1, H=16, S=300, name="frame1_det", state_std=0.05)
    x = device_inputs(w, DEV)
    args = (x["q"], x["k"], x["v"], x["gamma"], x["beta"])
    o1, s1 = F.frame_fwd(*args, x["state"])
    o2, s2 = F.frame_fwd(*args, x["state"])
    st = x["state"].clone()
    o3, _ = F.frame_fwd(*args, st, state_out=st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(o1, o3) and torch.equal(s1, st)


def test_single_frame_bf16_output_is_rounded_f32():
    w = CLIP_5S.with_(T=1, H=16, S=500, name="frame1_bf16out", state_std=0.05)
    x = device_inputs(w, DEV)
    args = (x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    o32, s32 = F.frame_fwd(*args)
    o16, s16 = F.frame_fwd(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(s16, s32)


def test_single_frame_key_scale_and_gates():
    """The key scale enters both launches (the prediction's keys and the
    update's): against the three-kernel path with the same scale.  With gates
    computed from activations, the gates are bit-identical on both paths."""
    w = CLIP_5S.with_(T=1, H=16, S=400, name="frame1_ks", state_std=0.05)
    x = device_inputs(w, DEV)
    ks = 1.0 / (128 * 400) ** 0.5
    raw_k = (x["k"].float() / ks).to(torch.bfloat16)
    (o1, s1), (o2, s2) = _both_paths(
        lambda: F.frame_fwd(x["q"], raw_k, x["v"], x["gamma"], x["beta"], x["state"], key_scale=ks))
    ro, rs = _rel(o1, o2), _rel(s1, s2)
    log(f"  key scale: relL2 O={ro:.3e} state={rs:.3e}")
    assert ro <= TOL and rs <= TOL  # each path is within 1e-5 of the oracle; a misplaced scale is O(1)

    g = torch.Generator(device="cpu").manual_seed(7)
    a = torch.randn((1, 16, 1, 400), generator=g).to(DEV)
    b = torch.randn((1, 16, 1, 400), generator=g).to(DEV)
    A_log = torch.randn(16, generator=g).to(DEV) * 0.5
    dt_bias = torch.randn(16, generator=g).to(DEV) * 0.5
    (r1, r2) = _both_paths(lambda: F.frame_fwd_gated(x["q"], x["k"], x["v"], a, b, A_log, dt_bias, x["state"]))
    o1, s1, g1, b1 = r1
    o2, s2, g2, b2 = r2
    assert torch.equal(g1, g2) and torch.equal(b1, b2)
    ro, rs = _rel(o1, o2), _rel(s1, s2)
    log(f"  gated: relL2 O={ro:.3e} state={rs:.3e}")
    assert ro <= TOL and rs <= TOL


def test_single_frame_switch_off_takes_three_kernel_path():
    w = CLIP_5S.with_(T=1, H=2, S=64)
    prev = F.set_single_frame(False)
    try:
        assert _path(w) == GDN_PATH_MFMA
    finally:
        F.set_single_frame(prev)
    assert _path(w) == GDN_PATH_FRAME
