"""GPU parity of the gate prologue (gdn_frame_fwd_gated): gamma_t, beta_t
computed from per-token gate pre-activations inside the build, keys scaled
inside the build, then the frame-wise GDN recurrence -- against the fp64
oracle (oracle/gate_ref.py) on the same seeded inputs, on the fused path and
on the separate-kernel paths.  Tolerances: relative L2 <= 2e-3 for bf16
inputs and 1e-5 for float32 inputs, for out, state_out and the gates."""
import ctypes

import numpy as np
import pytest
import torch

import frame_wise_gated_fwd_amd as F
from frame_wise_gated_fwd_amd._lib import Shape, GDN_BF16, GDN_F32
from synth import Workload, head_inputs, default_workers

from gpu_util import log, rel_l2, sample_frames

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gate_inputs(w, seed):
    """Per-token gate pre-activations and per-head parameters (seeded):
    a ~ N(-2, 1) so the mean decay stays near exp(-exp(A_log) softplus(-2)),
    b ~ N(0, 2); A_log ~ U(-1, 0.5), dt_bias ~ U(-1, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = (rng.standard_normal((w.B, w.H, w.T, w.S)) - 2.0).astype(np.float32)
    b = (rng.standard_normal((w.B, w.H, w.T, w.S)) * 2.0).astype(np.float32)
    A_log = rng.uniform(-1.0, 0.5, w.H).astype(np.float32)
    dt_bias = rng.uniform(-1.0, 1.0, w.H).astype(np.float32)
    return a, b, A_log, dt_bias


def _run(w, path_fused, frames=None, key_scale=None, odt=torch.float32):
    from oracle import gdn_head_gated
    log(f"gated {w.name}: B={w.B} H={w.H} T={w.T} S={w.S} D={w.D} {w.in_dtype} fused={path_fused}")
    ga, gb, A_log, dt_bias = _gate_inputs(w, w.seed + 1000)
    hs = [head_inputs(w, b, h) for b in range(w.B) for h in range(w.H)]
    tdt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32

    def stack(key):
        a = np.stack([d[key] for d in hs]).reshape((w.B, w.H) + hs[0][key].shape)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        return t.to(DEV)
    q, k, v = stack("q"), stack("k"), stack("v")
    state = stack("state") if hs[0]["state"] is not None else None
    ks = 1.0 if key_scale is None else key_scale
    prev = F.set_fused(path_fused)
    try:
        mfma = w.in_dtype == "bf16" and w.D == 128
        want = 2 if path_fused else 3 if mfma and w.T == 1 else 1 if mfma else 0  # 3: the single-frame kernel
        assert F.lib().gdn_path(ctypes.byref(Shape(w.B, w.H, w.T, w.S, w.D)),
                                GDN_BF16 if w.in_dtype == "bf16" else GDN_F32) == want
        out, st, gam, bet = F.frame_fwd_gated(q, k, v, torch.from_numpy(ga).to(DEV), torch.from_numpy(gb).to(DEV),
                                              torch.from_numpy(A_log).to(DEV), torch.from_numpy(dt_bias).to(DEV),
                                              state, key_scale=ks, out_dtype=odt)
        torch.cuda.synchronize()
    finally:
        F.set_fused(prev)
    fr = list(range(w.T)) if frames is None else list(frames)
    worst = {"O": 0.0, "state": 0.0, "gamma": 0.0, "beta": 0.0}
    for i, d in enumerate(hs):
        b, h = divmod(i, w.H)
        O, M, g, bt = gdn_head_gated(d["q"], d["k"], d["v"], ga[b, h], gb[b, h], A_log[h], dt_bias[h], d["state"],
                                     key_scale=ks, out_frames=fr)
        og = out[b, h, fr].float().cpu().numpy().astype(np.float64)
        for j in range(len(fr)):
            worst["O"] = max(worst["O"], rel_l2(og[j], O[j]))
        worst["state"] = max(worst["state"], rel_l2(st[b, h].cpu().numpy(), M))
        worst["gamma"] = max(worst["gamma"], rel_l2(gam[b, h].cpu().numpy(), g))
        worst["beta"] = max(worst["beta"], rel_l2(bet[b, h].cpu().numpy(), bt))
    log("  worst relL2 " + ", ".join(f"{k_}={v_:.3e}" for k_, v_ in worst.items()) + f" (tol {w.tol:g})")
    assert all(np.isfinite(x_) and x_ <= w.tol for x_ in worst.values()), worst
    return out, st, gam, bet


BASE = Workload(name="gated_clip", B=1, H=16, T=81, S=880, D=128, in_dtype="bf16", seed=81,
                gamma_range=(0.95, 1.0), beta_kind="sigmoid_normal", state_std=0.02, keys_prescaled=False)


def test_gated_fused_5s_raw_keys():
    """The 5 s clip shape (16 heads, 81 frames, 880 tokens) on the fused path,
    raw keys with the pages' scale 1/sqrt(D*S) applied in the build."""
    w = BASE
    _run(w, True, frames=sample_frames(w.T, seed=1), key_scale=w.key_scale)


def test_gated_fused_equals_separate_kernels_bitwise():
    """The build items' gates and the gate kernel's are the same float32
    values; the fused kernel and the three-kernel schedule then agree bit
    for bit, as gdn_frame_fwd's paths do (20 heads: two launch groups, the
    parameters indexed by head within the batch element; B = 2)."""
    w = BASE.with_(name="gated_b2", B=2, H=10, T=70, S=300, keys_prescaled=True)
    o1, s1, g1, b1 = _run(w, True, frames=[0, 35, 69])
    o2, s2, g2, b2 = _run(w, False, frames=[0, 35, 69])
    assert torch.equal(g1, g2) and torch.equal(b1, b2)
    assert torch.equal(s1, s2) and torch.equal(o1, o2)


@pytest.mark.parametrize("T,S,D,dt", [(1, 880, 128, "bf16"), (5, 17, 128, "bf16"), (6, 40, 64, "bf16"),
                                      (4, 33, 32, "f32")])
def test_gated_separate_kernel_paths(T, S, D, dt):
    w = BASE.with_(name=f"gated_{T}_{S}_{D}_{dt}", H=3, T=T, S=S, D=D, in_dtype=dt, keys_prescaled=True,
                   tol=1e-5 if dt == "f32" else 2e-3)
    _run(w, False)
