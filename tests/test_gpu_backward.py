"""GPU parity of the backward pass (gdn_frame_bwd, through the C ABI) against
the fp64 backward oracle on the same seeded inputs, plus consistency checks
that hold bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import frame_wise_gated_fwd_amd as F
from synth import CLIP_5S, Workload, head_inputs
from gpu_util import device_inputs, RelL2, log, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KEYS = ("dq", "dk", "dv", "dgamma", "dbeta", "dstate")


def _upstream(w, seed, with_dstate):
    """Seeded incoming gradients: d_out bf16 (as the inputs), d_state_out f32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    d_out = rng.standard_normal((w.B, w.H, w.T, w.S, w.D), dtype=np.float32)
    d_out_t = torch.from_numpy(d_out).to(torch.bfloat16)
    d_state = (rng.standard_normal((w.B, w.H, w.D, w.D), dtype=np.float32) * 0.1) if with_dstate else None
    return d_out_t, d_state


def _gpu_backward(x, d_out_t, d_state):
    ds = None if d_state is None else torch.from_numpy(d_state).to(DEV)
    return dict(zip(KEYS, F.frame_bwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], d_out_t.to(DEV),
                                      x["state"], ds)))


def _backward_parity(w, seed=1, with_dstate=True, heads=None, tol=2e-3):
    log(f"backward {w.name}: B={w.B} H={w.H} T={w.T} S={w.S} D={w.D} d_state={with_dstate}")
    x = device_inputs(w, DEV)
    d_out_t, d_state = _upstream(w, seed, with_dstate)
    got = _gpu_backward(x, d_out_t, d_state)
    torch.cuda.synchronize()
    d_out_bits = d_out_t.view(torch.int16).numpy().view(np.uint16)
    hs = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    err = {k: RelL2() for k in KEYS}
    for b, h in hs:
        d = head_inputs(w, b, h)
        ref = oracle.gdn_head_backward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d.get("state"),
                                       d_out_bits[b, h], None if d_state is None else d_state[b, h])
        for key in KEYS:
            err[key].add(got[key][b, h].cpu().numpy(), ref[key])
    log("  relL2 " + ", ".join(f"{k}={err[k].value:.2e}" for k in KEYS))
    for key in KEYS:
        assert np.isfinite(err[key].value) and err[key].value <= tol, (key, err[key].value)
    return x, d_out_t, d_state, got


def test_backward_small_ragged():
    w = Workload(name="bwd_small", B=1, H=3, T=7, S=100, D=128, in_dtype="bf16", seed=71,
                 gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal", state_std=0.05)
    _backward_parity(w)


@pytest.mark.parametrize("T", [1, 64, 65])
def test_backward_segment_boundaries(T):
    """A single frame; 64 frames (one segment); 65 frames (two segments)."""
    w = Workload(name=f"bwd_t{T}", B=1, H=4, T=T, S=24, D=128, in_dtype="bf16", seed=76 + T,
                 gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal", state_std=0.05)
    _backward_parity(w)


def test_backward_zero_state_no_state_gradient():
    w = Workload(name="bwd_zero", B=2, H=2, T=5, S=37, D=128, in_dtype="bf16", seed=72,
                 gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal")
    _backward_parity(w, with_dstate=False)


def test_backward_clip_frames_sampled_heads():
    w = CLIP_5S.with_(T=12, name="bwd_clip_t12", state_std=0.02)
    _backward_parity(w, heads=[(0, 0), (0, 5), (0, 10), (0, 15)])


def test_backward_in_place_state_gradient_and_determinism():
    w = Workload(name="bwd_inplace", B=1, H=4, T=6, S=64, D=128, in_dtype="bf16", seed=73,
                 gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal", state_std=0.05)
    x = device_inputs(w, DEV)
    d_out_t, d_state = _upstream(w, 5, True)
    a = _gpu_backward(x, d_out_t, d_state)
    b = _gpu_backward(x, d_out_t, d_state)
    ds = torch.from_numpy(d_state).to(DEV)
    res = F.frame_bwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], d_out_t.to(DEV), x["state"], ds,
                      d_state_in=ds)
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(a[key], b[key]), key
    assert res[5] is ds and torch.equal(ds, a["dstate"])
    for i, key in enumerate(KEYS[:5]):
        assert torch.equal(res[i], a[key]), key


def test_backward_stress_slice():
    """Two heads of the stress workload (gamma ~ U(0.999, 1), beta ~ U(0.9, 1),
    a tenth of the key rows x4), 70 frames: two segments, zero initial state."""
    from synth import STRESS_B4
    w = STRESS_B4.with_(name="bwd_stress_slice", B=1, H=2, T=70)
    _backward_parity(w)


def test_backward_seq60s_full_size_sampled_heads():
    """The 60 s workload at full size, in the configuration bench.py times
    (one call over all 16 heads and 961 frames, 3 segments); two heads are
    checked whole against the oracle.  d_out and d_state_out are drawn on the
    device (seeded) and the checked heads' values copied back for the oracle."""
    from synth import SEQ_60S
    w = SEQ_60S
    log(f"backward {w.name}: B={w.B} H={w.H} T={w.T} S={w.S} D={w.D} (full size, 2 heads checked)")
    x = device_inputs(w, DEV)
    gen = torch.Generator(device=DEV).manual_seed(11)
    d_out = torch.randn((w.B, w.H, w.T, w.S, w.D), generator=gen, device=DEV).to(torch.bfloat16)
    d_state = torch.randn((w.B, w.H, w.D, w.D), generator=gen, device=DEV) * 0.1
    got = dict(zip(KEYS, F.frame_bwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], d_out, x["state"], d_state)))
    torch.cuda.synchronize()
    err = {k: RelL2() for k in KEYS}
    for b, h in [(0, 3), (0, 12)]:
        d = head_inputs(w, b, h)
        dob = d_out[b, h].cpu().view(torch.int16).numpy().view(np.uint16)
        ref = oracle.gdn_head_backward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d.get("state"), dob,
                                       d_state[b, h].cpu().numpy())
        for key in KEYS:
            err[key].add(got[key][b, h].cpu().numpy(), ref[key])
    log("  relL2 " + ", ".join(f"{k}={err[k].value:.2e}" for k in KEYS))
    for key in KEYS:
        assert np.isfinite(err[key].value) and err[key].value <= 2e-3, (key, err[key].value)


def test_backward_segmented_schedule():
    """T = 150 is cut into segments (the forward recomputation and the
    reverse-time pass run segment by segment on the side streams)."""
    w = Workload(name="bwd_segments", B=1, H=3, T=150, S=48, D=128, in_dtype="bf16", seed=75,
                 gamma_range=(0.95, 1.0), beta_kind="sigmoid_normal", state_std=0.05)
    _backward_parity(w)


@pytest.mark.parametrize("T,t0,S", [(9, 4, 120), (150, 70, 40)])
def test_chunked_backward_equals_one_call_bitwise(T, t0, S):
    """Frames [t0, T) then [0, t0), carrying the forward state forwards and the
    state gradient backwards, reproduce the one-call backward bit for bit
    (the calls also differ in how many segments their schedules use)."""
    w = Workload(name="bwd_chunks", B=1, H=3, T=T, S=S, D=128, in_dtype="bf16", seed=74,
                 gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal", state_std=0.05)
    log(f"chunked backward: T={T} t0={t0} S={S}")
    x = device_inputs(w, DEV)
    d_out_t, d_state = _upstream(w, 6, True)
    one = _gpu_backward(x, d_out_t, d_state)
    sl1, sl2 = slice(0, t0), slice(t0, w.T)
    part = lambda key, sl: x[key][:, :, sl].contiguous()
    _, mid = F.frame_fwd(part("q", sl1), part("k", sl1), part("v", sl1), part("gamma", sl1),
                         part("beta", sl1), x["state"])
    d_out = d_out_t.to(DEV)
    g2 = F.frame_bwd(part("q", sl2), part("k", sl2), part("v", sl2), part("gamma", sl2), part("beta", sl2),
                     d_out[:, :, sl2].contiguous(), mid, torch.from_numpy(d_state).to(DEV))
    g1 = F.frame_bwd(part("q", sl1), part("k", sl1), part("v", sl1), part("gamma", sl1), part("beta", sl1),
                     d_out[:, :, sl1].contiguous(), x["state"], g2[5])
    torch.cuda.synchronize()
    for i, key in enumerate(("dq", "dk", "dv", "dgamma", "dbeta")):
        assert torch.equal(torch.cat([g1[i], g2[i]], dim=2), one[key]), key
    assert torch.equal(g1[5], one["dstate"])


def test_backward_rejects_unsupported():
    q = torch.zeros((1, 1, 2, 8, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.ones((1, 1, 2), device=DEV)
    with pytest.raises(F.GDNError):
        F.frame_bwd(q, q, q, g, g, q)


@pytest.mark.parametrize("B,H,T,S", [(0, 2, 3, 8), (1, 3, 0, 8), (1, 3, 5, 0), (2, 1, 70, 0)])
def test_backward_empty_shapes(B, H, T, S):
    """No heads: nothing.  No frames: d_state_in = d_state_out.  Frames
    without tokens: the backward of the pure decay (dbeta = 0) against the
    backward oracle; also in place."""
    D = 128
    log(f"backward empty shape B={B} H={H} T={T} S={S}")
    rng = np.random.Generator(np.random.PCG64(200 + T + S))
    e = torch.empty((B, H, T, S, D), dtype=torch.bfloat16, device=DEV)
    gamma = rng.uniform(0.5, 1.0, (B, H, T)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (B, H, T)).astype(np.float32)
    st = (rng.standard_normal((B, H, D, D)) * 0.1).astype(np.float32)
    ds = rng.standard_normal((B, H, D, D)).astype(np.float32)
    g_t, b_t = torch.from_numpy(gamma).to(DEV), torch.from_numpy(beta).to(DEV)
    for with_state, in_place in ((True, False), (False, False), (True, True)):
        s_in = torch.from_numpy(st).to(DEV) if with_state else None
        d_so = torch.from_numpy(ds).to(DEV)
        kw = {"d_state_in": d_so} if in_place else {}
        got = dict(zip(KEYS, F.frame_bwd(e, e, e, g_t, b_t, e, s_in, d_so, **kw)))
        torch.cuda.synchronize()
        assert got["dq"].shape == (B, H, T, S, D) and got["dstate"].shape == (B, H, D, D)
        if B * H == 0:
            continue
        if T == 0:
            assert torch.equal(got["dstate"].cpu(), torch.from_numpy(ds))
            continue
        assert torch.equal(got["dbeta"].cpu(), torch.zeros((B, H, T)))
        for b in range(B):
            for h in range(H):
                z = np.zeros((T, S, D))
                ref = oracle.gdn_head_backward(z, z, z, gamma[b, h], beta[b, h], st[b, h] if with_state else None,
                                               z, ds[b, h])
                assert rel_l2(got["dstate"][b, h].cpu().numpy(), ref["dstate"]) <= 1e-6
                if with_state:
                    assert rel_l2(got["dgamma"][b, h].cpu().numpy(), ref["dgamma"]) <= 1e-4
                else:
                    assert torch.equal(got["dgamma"][b, h].cpu(), torch.zeros(T))
