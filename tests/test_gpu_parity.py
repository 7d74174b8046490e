"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Tolerances: relative L2 <= 1e-5 for float32 inputs and
<= 2e-3 for bf16 inputs with float32 accumulation, for the output and for the
final state.  Stage tests hold float32-accumulation arithmetic to 1e-5."""
import numpy as np
import pytest
import torch

import oracle
import frame_wise_gated_fwd_amd as F
from synth import TINY_F32, CLIP_5S, SEQ_60S, STREAM_60S, STRESS_B4, Workload, head_inputs

from gpu_util import device_inputs, oracle_heads, RelL2, rel_l2, sample_frames, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy().astype(np.float64)


def _bf16(a: np.ndarray) -> torch.Tensor:
    from synth import f32_to_bf16_bits
    return torch.from_numpy(f32_to_bf16_bits(a.astype(np.float32)).view(np.int16)).view(torch.bfloat16)


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# stage 1: G_t = K^T K, U_t = V^T K
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,T,S,D,dt", [
    (1, 2, 3, 880, 128, "bf16"),     # MFMA path, full frame
    (1, 1, 2, 100, 128, "bf16"),     # MFMA path, ragged token tail (100 = 64 + 36)
    (1, 1, 2, 1, 128, "bf16"),       # single token
    (1, 2, 3, 37, 64, "bf16"),       # plain path
    (1, 2, 2, 16, 32, "f32"),        # plain path, float32
    (2, 1, 2, 70, 112, "f32"),
])
def test_build_maps_stage(B, H, T, S, D, dt):
    log(f"build_maps B={B} H={H} T={T} S={S} D={D} {dt}")
    rng = np.random.Generator(np.random.PCG64(S * 1000 + D))
    k = (rng.standard_normal((B, H, T, S, D)) / np.sqrt(D * S)).astype(np.float32)
    v = rng.standard_normal((B, H, T, S, D)).astype(np.float32)
    if dt == "bf16":
        kt, vt = _bf16(k), _bf16(v)
    else:
        kt, vt = torch.from_numpy(k), torch.from_numpy(v)
    G, U = F.build_maps(kt.to(DEV), vt.to(DEV))
    torch.cuda.synchronize()
    kx, vx = _to_np(kt), _to_np(vt)
    rg, ru = RelL2(), RelL2()
    for b in range(B):
        for h in range(H):
            Gr, Ur = oracle.build_maps_head(kx[b, h], vx[b, h])
            rg.add(_to_np(G[b, h]), Gr)
            ru.add(_to_np(U[b, h]), Ur)
    log(f"  relL2 G={rg.value:.3e} U={ru.value:.3e}")
    assert rg.value <= 1e-5 and ru.value <= 1e-5


# ---------------------------------------------------------------------------
# stage 2: the state pass
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("H,T,D,with_state", [(3, 40, 128, True), (2, 17, 128, False),
                                              (2, 9, 64, True), (1, 5, 32, False)])
def test_state_pass_stage(H, T, D, with_state):
    log(f"state_pass H={H} T={T} D={D} state={with_state}")
    rng = np.random.Generator(np.random.PCG64(T * 100 + D))
    S = 200
    k = rng.standard_normal((1, H, T, S, D)) / np.sqrt(D * S)
    v = rng.standard_normal((1, H, T, S, D))
    G = np.einsum("bhtsi,bhtsj->bhtij", k, k).astype(np.float32)
    U = np.einsum("bhtsi,bhtsj->bhtij", v, k).astype(np.float32)
    gamma = rng.uniform(0.9, 1.0, (1, H, T)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (1, H, T)).astype(np.float32)
    st = (rng.standard_normal((1, H, D, D)) * 0.1).astype(np.float32) if with_state else None
    M_all, so = F.state_pass(*(torch.from_numpy(a).to(DEV) for a in (G, U, gamma, beta)),
                             None if st is None else torch.from_numpy(st).to(DEV))
    torch.cuda.synchronize()
    rm, rs = RelL2(), RelL2()
    for h in range(H):
        ref = oracle.state_pass_head(G[0, h], U[0, h], gamma[0, h], beta[0, h],
                                     None if st is None else st[0, h])
        rm.add(_to_np(M_all[0, h]), ref)
        rs.add(_to_np(so[0, h]), ref[-1])
    log(f"  relL2 M_all={rm.value:.3e} state={rs.value:.3e}")
    assert rm.value <= 1e-5 and rs.value <= 1e-5


# ---------------------------------------------------------------------------
# stage 3: the output
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,S,D,dt,odt", [(3, 880, 128, "bf16", "f32"), (2, 45, 128, "bf16", "f32"),
                                          (2, 130, 128, "bf16", "bf16"), (2, 70, 64, "bf16", "f32"),
                                          (2, 33, 48, "f32", "f32")])
def test_output_stage(T, S, D, dt, odt):
    log(f"output T={T} S={S} D={D} in={dt} out={odt}")
    rng = np.random.Generator(np.random.PCG64(S + D))
    H = 2
    q = rng.standard_normal((1, H, T, S, D)).astype(np.float32)
    M = rng.standard_normal((1, H, T, D, D)).astype(np.float32)
    qt = _bf16(q) if dt == "bf16" else torch.from_numpy(q)
    out_dtype = torch.bfloat16 if odt == "bf16" else torch.float32
    O = F.output(qt.to(DEV), torch.from_numpy(M).to(DEV), out_dtype)
    torch.cuda.synchronize()
    qx = _to_np(qt)
    r = RelL2()
    for h in range(H):
        r.add(_to_np(O[0, h]), oracle.output_head(qx[0, h], M[0, h]))
    # a bf16 output is float32 arithmetic followed by one rounding (<= 2^-9 relative)
    tol = 2.0 ** -9 * 1.01 + 1e-5 if odt == "bf16" else 1e-5
    log(f"  relL2 O={r.value:.3e} (tol {tol:.2e})")
    assert r.value <= tol


# ---------------------------------------------------------------------------
# the whole forward on the seeded workloads
# ---------------------------------------------------------------------------
def _forward_parity(w: Workload, frames=None, heads=None, chunks=None, workspace=None):
    """Run the GPU forward on w (optionally streamed in `chunks`), compare O at
    `frames` (all when None) for `heads` (all when None) and the final state."""
    log(f"workload {w.name}: B={w.B} H={w.H} T={w.T} S={w.S} D={w.D} {w.in_dtype}"
        f"{' streamed ' + str(len(chunks)) + ' calls' if chunks else ''}")
    x = device_inputs(w, DEV)
    log("  inputs on device")
    if chunks:
        out = torch.empty(x["q"].shape, dtype=torch.float32, device=DEV)
        state = x["state"].clone() if x["state"] is not None else \
            torch.zeros((w.B, w.H, w.D, w.D), dtype=torch.float32, device=DEV)
        t0 = 0
        for c in chunks:
            sl = slice(t0, t0 + c)
            o, _ = F.frame_fwd(x["q"][:, :, sl].contiguous(), x["k"][:, :, sl].contiguous(),
                               x["v"][:, :, sl].contiguous(), x["gamma"][:, :, sl].contiguous(),
                               x["beta"][:, :, sl].contiguous(), state, state_out=state)
            out[:, :, sl] = o
            t0 += c
        st = state
    else:
        out, st = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"], workspace=workspace)
    torch.cuda.synchronize()
    log("  GPU forward done")
    hs = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    ro, rs = RelL2(), RelL2()
    worst_frame = worst_state = 0.0  # the largest relL2 of any one frame of any head, of any head's state
    for b, h, O, M in oracle_heads(w, hs, frames):
        og = _to_np(out[b, h] if frames is None else out[b, h, list(frames)])
        ro.add(og, O)
        sg = _to_np(st[b, h])
        rs.add(sg, M)
        for i in range(len(O)):
            worst_frame = max(worst_frame, rel_l2(og[i], O[i]))
        worst_state = max(worst_state, rel_l2(sg, M))
    log(f"  relL2 O={ro.value:.3e} state={rs.value:.3e} (tol {w.tol:g}); max|dO|={ro.max_abs:.3e}; "
        f"worst frame {worst_frame:.3e}, worst head state {worst_state:.3e}")
    assert np.isfinite(ro.value) and np.isfinite(rs.value)
    assert ro.value <= w.tol and rs.value <= w.tol
    # every frame and every head's state on its own, not only the whole tensor
    assert worst_frame <= w.tol and worst_state <= w.tol
    return out, st, x


def test_forward_tiny_f32():
    _forward_parity(TINY_F32)


def test_forward_clip5s_bf16():
    _forward_parity(CLIP_5S)


def test_forward_seq60s_full_size():
    """The 60 s workload on the fused path with exactly the workspace the
    library asks for (its rings, not the whole sequence's maps)."""
    import ctypes
    from frame_wise_gated_fwd_amd._lib import Shape, GDN_BF16, GDN_PATH_FUSED
    w = SEQ_60S
    shp = Shape(w.B, w.H, w.T, w.S, w.D)
    L = F.lib()
    assert L.gdn_path(ctypes.byref(shp), GDN_BF16) == GDN_PATH_FUSED
    need = L.gdn_workspace_bytes(ctypes.byref(shp), GDN_BF16)
    assert need == L.gdn_path_workspace_bytes(ctypes.byref(shp), GDN_BF16, GDN_PATH_FUSED)
    assert need <= 80 << 20
    log(f"  workspace {need / 2**20:.1f} MiB")
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    _forward_parity(w, frames=sample_frames(w.T, seed=3), workspace=ws)


@pytest.fixture
def mfma_single_frames():
    """Single-frame calls through the three-kernel path, which sums a frame's
    tokens in the same order as a longer call."""
    prev = F.set_single_frame(False)
    yield
    F.set_single_frame(prev)


def test_forward_stream60s_matches_single_call(mfma_single_frames):
    """24 calls of 40 frames and one of a single frame, the state carried in
    place, against one call: same kernels and arithmetic, bit for bit (the
    single frame through the three-kernel path; the single-frame kernels are
    checked against the oracle below)."""
    w = STREAM_60S
    out_s, st_s, x = _forward_parity(w, frames=sample_frames(w.T, seed=4), chunks=w.stream_chunks)
    out1, st1 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    torch.cuda.synchronize()
    # same kernels, same arithmetic, state handed over in float32: bit-identical
    assert torch.equal(out_s, out1)
    assert torch.equal(st_s, st1)


def test_checkpoint_resume_is_bitwise(tmp_path):
    """A chunk-causal rollout stopped after 70 of 161 frames: state_out goes
    to disk (a float32 .npy file), every device buffer is dropped, the state
    is loaded back into a fresh tensor and the rollout continues; out and the
    final state equal one uninterrupted call bit for bit (the state is the
    whole memory of the recurrence and crosses the file exactly)."""
    import os
    w = CLIP_5S.with_(T=161, H=16, S=200, name="clip_t161_resume", state_std=0.02)
    x = device_inputs(w, DEV)
    out1, st1 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    cut = 70
    a = {k_: x[k_][:, :, :cut].contiguous() for k_ in ("q", "k", "v", "gamma", "beta")}
    o_a, st_a = F.frame_fwd(a["q"], a["k"], a["v"], a["gamma"], a["beta"], x["state"])
    torch.cuda.synchronize()
    path = os.path.join(tmp_path, "state.npy")
    np.save(path, st_a.cpu().numpy())
    o_a = o_a.cpu()
    del a, st_a
    torch.cuda.empty_cache()
    state = torch.from_numpy(np.load(path)).to(DEV)
    b = {k_: x[k_][:, :, cut:].contiguous() for k_ in ("q", "k", "v", "gamma", "beta")}
    o_b, st_b = F.frame_fwd(b["q"], b["k"], b["v"], b["gamma"], b["beta"], state)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o_a, o_b.cpu()], dim=2), out1.cpu())
    assert torch.equal(st_b, st1)


def test_forward_stress_b4_all_heads():
    """All 64 heads' final states, and each head's output at 15 sampled
    frames.  A launch covers the 16 heads of one batch element, head h on
    XCD h % 8 in head slot h // 8, so every XCD and both slots are checked
    in each of the four launches."""
    w = STRESS_B4
    _forward_parity(w, frames=sample_frames(w.T, seed=5))


# ---------------------------------------------------------------------------
# the segmented, multi-stream schedule of the MFMA path
# ---------------------------------------------------------------------------
@pytest.fixture
def three_kernel_path():
    """Route long sequences through the three-kernel segmented schedule."""
    prev = F.set_fused(False)
    yield
    F.set_fused(prev)


def test_segmented_forward_equals_stage_chain_bitwise(three_kernel_path):
    """T = 330 runs as 6 overlapped segments on three streams, their maps in
    three workspace slots that each serve two segments (exactly the
    workspace the library asks for); the stage entry points run each kernel
    once over all frames on one stream, exchanging float32 row-major maps.
    Both feed the MFMAs the same bf16 hi/lo operands, so the results agree
    bit for bit."""
    import ctypes
    from frame_wise_gated_fwd_amd._lib import Shape, GDN_BF16, GDN_PATH_MFMA
    w = CLIP_5S.with_(T=330, H=3, S=200, name="clip_t330_s200", state_std=0.02)
    shp = Shape(w.B, w.H, w.T, w.S, w.D)
    L = F.lib()
    assert L.gdn_path(ctypes.byref(shp), GDN_BF16) == GDN_PATH_MFMA
    need = L.gdn_workspace_bytes(ctypes.byref(shp), GDN_BF16)
    assert need == 9 * 3 * 55 * 65536  # 6 segments of 55 frames, three held at once
    x = device_inputs(w, DEV)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out, st = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"], workspace=ws)
    G, U = F.build_maps(x["k"], x["v"])
    M_all, st2 = F.state_pass(G, U, x["gamma"], x["beta"], x["state"])
    out2 = F.output(x["q"], M_all)
    torch.cuda.synchronize()
    assert torch.equal(st, st2)
    assert torch.equal(out, out2)


def test_fused_kernel_equals_three_kernel_path_bitwise():
    """The fused kernel (one launch, rings on chip) and the
    three-kernel schedule run the same per-element arithmetic: identical
    results on the 5 s workload (16 heads, 81 frames) and on 20 heads (two
    head groups, the second partial) with a bf16 output."""
    import ctypes
    from frame_wise_gated_fwd_amd._lib import Shape, lib, GDN_BF16
    for w, odt in ((CLIP_5S.with_(state_std=0.02, name="clip5s_state"), torch.float32),
                   (CLIP_5S.with_(H=20, T=70, S=300, name="clip_h20", state_std=0.02), torch.bfloat16)):
        assert lib().gdn_path(ctypes.byref(Shape(w.B, w.H, w.T, w.S, w.D)), GDN_BF16) == 2
        x = device_inputs(w, DEV)
        o1, s1 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"], out_dtype=odt)
        prev = F.set_fused(False)
        try:
            o2, s2 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"], out_dtype=odt)
        finally:
            F.set_fused(prev)
        torch.cuda.synchronize()
        assert torch.equal(s1, s2) and torch.equal(o1, o2), w.name


def test_single_frame_calls_equal_one_call_bitwise(mfma_single_frames):
    """Launches of a few frames take the small-launch kernels (a build with
    more loads in flight, an output split over token parts); 12 successive
    T=1 calls must reproduce one T=12 call (16 x 12 frames, full-size
    kernels) bit for bit, and match the oracle."""
    w = CLIP_5S.with_(T=12, name="clip_t12", state_std=0.02)
    x = device_inputs(w, DEV)
    out1, st1 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    state = x["state"].clone()
    outs = []
    for t in range(w.T):
        sl = slice(t, t + 1)
        o, _ = F.frame_fwd(x["q"][:, :, sl].contiguous(), x["k"][:, :, sl].contiguous(),
                           x["v"][:, :, sl].contiguous(), x["gamma"][:, :, sl].contiguous(),
                           x["beta"][:, :, sl].contiguous(), state, state_out=state)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=2), out1)
    assert torch.equal(state, st1)
    _forward_parity(w, frames=[0, 5, 11])


def test_small_launch_threshold_is_bitwise():
    """128 head-frames take the small-launch kernels (each frame's build over
    four workgroups, its output over token parts), 136 the full-size ones:
    the 16 heads the two launches share agree bit for bit."""
    w = CLIP_5S.with_(H=17, T=8, S=300, name="clip_h17_t8", state_std=0.02)
    x = device_inputs(w, DEV)
    full_out, full_st = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    sub = {n: x[n][:, :16].contiguous() for n in ("q", "k", "v", "gamma", "beta", "state")}
    few_out, few_st = F.frame_fwd(sub["q"], sub["k"], sub["v"], sub["gamma"], sub["beta"], sub["state"])
    torch.cuda.synchronize()
    assert torch.equal(few_out, full_out[:, :16]) and torch.equal(few_st, full_st[:, :16])


@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16])
def test_single_frame_launch_is_bitwise(odt, mfma_single_frames):
    """A single-frame call's output equals the first frame of a two-frame
    call, for either output type, and its state equals the stage entry
    points' (float32 maps, 32-row state pass)."""
    w = CLIP_5S.with_(T=2, S=300, name="clip_t2_s300", state_std=0.02)
    x = device_inputs(w, DEV)
    two_out, _ = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"], out_dtype=odt)
    one = {n: x[n][:, :, :1].contiguous() for n in ("q", "k", "v", "gamma", "beta")}
    one_out, one_st = F.frame_fwd(one["q"], one["k"], one["v"], one["gamma"], one["beta"], x["state"],
                                  out_dtype=odt)
    st_ref = F.state_pass(*F.build_maps(one["k"], one["v"]), one["gamma"], one["beta"], x["state"])[1]
    torch.cuda.synchronize()
    assert torch.equal(one_out, two_out[:, :, :1])
    assert torch.equal(one_st, st_ref)


@pytest.mark.parametrize("fused", [True, False])
def test_forward_is_ordered_on_a_user_stream(fused):
    """Work queued on the caller's stream before the call is seen by the
    whole call (every segment, or the fused kernel), and work queued after
    it runs after the call's last kernel."""
    prev = F.set_fused(fused)
    try:
        _ordered_on_user_stream()
    finally:
        F.set_fused(prev)


def _ordered_on_user_stream():
    w = CLIP_5S.with_(T=140, H=3, S=200, name="clip_t140_s200", state_std=0.02)
    x = device_inputs(w, DEV)
    ref_o, ref_s = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(2):
            q = torch.zeros_like(x["q"])
            q.copy_(x["q"])                  # produced on s just before the call
            o, st = F.frame_fwd(q, x["k"], x["v"], x["gamma"], x["beta"], x["state"])
            q.fill_(float("nan"))            # overwritten on s right after it
            o_copy = o.clone()
    s.synchronize()
    assert torch.equal(o_copy, ref_o) and torch.equal(st, ref_s)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,S,D,dt", [(1, 880, 128, "bf16"), (5, 1, 128, "bf16"), (4, 17, 128, "bf16"),
                                      (3, 130, 16, "bf16"), (3, 50, 112, "bf16"), (2, 8, 64, "f32"),
                                      (6, 100, 128, "f32")])
def test_forward_edge_shapes(T, S, D, dt):
    w = Workload(name=f"edge_{T}_{S}_{D}_{dt}", B=2, H=2, T=T, S=S, D=D, in_dtype=dt, seed=40 + T + S,
                 gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal", state_std=0.05,
                 tol=1e-5 if dt == "f32" else 2e-3)
    _forward_parity(w)


@pytest.mark.parametrize("B,H,T,S,state", [
    (1, 3, 33, 880, True),     # just long enough for the fused kernel; 5 of 8 XCDs without a head
    (1, 17, 70, 100, True),    # two launch groups, the second with one head; ragged tokens (64 + 36)
    (2, 4, 67, 1, False),      # one token per frame (3 of the 4 parts of a tail output empty), zero state
    (1, 8, 66, 17, True),      # one head per XCD, 17 tokens
])
def test_fused_kernel_edge_shapes(B, H, T, S, state):
    import ctypes
    from frame_wise_gated_fwd_amd._lib import Shape, lib, GDN_BF16
    assert lib().gdn_path(ctypes.byref(Shape(B, H, T, S, 128)), GDN_BF16) == 2
    w = Workload(name=f"fused_{B}_{H}_{T}_{S}", B=B, H=H, T=T, S=S, D=128, in_dtype="bf16",
                 seed=60 + H + T + S, gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal",
                 state_std=0.05 if state else None)
    _forward_parity(w, frames=sample_frames(T, seed=T))


def test_fused_kernel_bf16_output_matches_rounded_f32():
    w = CLIP_5S.with_(T=66, H=5, S=300, name="clip_t66_h5", state_std=0.02)
    x = device_inputs(w, DEV)
    o32, s32 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    o16, s16 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(s32, s16)
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_forward_bf16_output():
    w = CLIP_5S.with_(T=7, name="clip_t7")
    x = device_inputs(w, DEV)
    o32, s32 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"])
    o16, s16 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(s32, s16)
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_zero_state_equals_none_and_in_place_state():
    w = CLIP_5S.with_(T=6, name="clip_t6", state_std=0.02)
    x = device_inputs(w, DEV)
    z = torch.zeros_like(x["state"])
    o1, s1 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], None)
    o2, s2 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], z)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    ref_o, ref_s = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    st = x["state"].clone()
    o3, s3 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], st, state_out=st)
    torch.cuda.synchronize()
    assert s3.data_ptr() == st.data_ptr()
    assert torch.equal(o3, ref_o) and torch.equal(st, ref_s)


def test_deterministic_bitwise():
    w = CLIP_5S.with_(T=12, name="clip_t12")
    x = device_inputs(w, DEV)
    a = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"])
    b = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_nan_propagates_within_its_head_only():
    w = CLIP_5S.with_(T=5, H=2, name="clip_nan")
    x = device_inputs(w, DEV)
    x["k"][0, 1, 2, 7, 3] = float("nan")
    o, s = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"])
    torch.cuda.synchronize()
    assert torch.isfinite(o[0, 0]).all() and torch.isfinite(s[0, 0]).all()
    assert torch.isfinite(o[0, 1, :2]).all()
    assert torch.isnan(o[0, 1, 2:]).any() and torch.isnan(s[0, 1]).any()


def test_binding_rejects_bad_arguments():
    q = torch.zeros((1, 1, 2, 16, 128), dtype=torch.bfloat16, device=DEV)
    g = torch.ones((1, 1, 2), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        F.frame_fwd(q, q, q[:, :, :1].contiguous(), g, g)
    with pytest.raises(TypeError):
        F.frame_fwd(q, q.float(), q, g, g)
    with pytest.raises(F.GDNError):
        bad = torch.zeros((1, 1, 2, 16, 100), dtype=torch.bfloat16, device=DEV)
        F.frame_fwd(bad, bad, bad, g, g)


def test_timed_entry_point_matches_and_reports():
    import ctypes
    from frame_wise_gated_fwd_amd._lib import Shape, lib, GDN_BF16, GDN_F32
    w = CLIP_5S.with_(T=9, name="clip_t9", state_std=0.02)
    x = device_inputs(w, DEV)
    ref_o, ref_s = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    L = lib()
    shp = Shape(w.B, w.H, w.T, w.S, w.D)
    wsb = L.gdn_workspace_bytes(ctypes.byref(shp), GDN_BF16)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(ref_o)
    so = torch.empty_like(ref_s)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    ms, nl = (ctypes.c_float * 3)(), (ctypes.c_int * 3)()
    st = L.gdn_frame_fwd_timed(ctypes.byref(shp), GDN_BF16, GDN_F32, P(x["q"]), P(x["k"]), P(x["v"]),
                               P(x["gamma"]), P(x["beta"]), P(x["state"]), P(out), P(so), P(ws), wsb,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ms, nl)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(so, ref_s)
    path = L.gdn_path(ctypes.byref(shp), GDN_BF16)
    assert path == 1
    assert list(nl) == [1, 1, 1] and all(m > 0 for m in ms)


# ---------------------------------------------------------------------------
# empty shapes: no heads, no frames, frames without tokens
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,T,S,D,dt", [(0, 2, 3, 8, 128, "bf16"), (1, 0, 3, 8, 64, "f32"),
                                          (1, 3, 0, 8, 128, "bf16"), (2, 2, 0, 5, 32, "f32"),
                                          (1, 3, 4, 0, 128, "bf16"), (2, 2, 5, 0, 48, "f32"),
                                          (1, 2, 70, 0, 128, "bf16")])
def test_empty_shapes(B, H, T, S, D, dt):
    """T = 0 leaves the state; S = 0 decays it, M_t = gamma_t M_{t-1} (one
    float32 product per frame, so it equals the same products in numpy bit
    for bit); B*H = 0 does nothing.  Against the oracle as well."""
    log(f"empty shape B={B} H={H} T={T} S={S} D={D} {dt}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    rng = np.random.Generator(np.random.PCG64(100 + T + S + D))
    qkv = torch.empty((B, H, T, S, D), dtype=tdt, device=DEV)
    gamma = rng.uniform(0.5, 1.0, (B, H, T)).astype(np.float32)
    beta = rng.uniform(-0.5, 1.5, (B, H, T)).astype(np.float32)
    st = rng.standard_normal((B, H, D, D)).astype(np.float32)
    g_t, b_t = torch.from_numpy(gamma).to(DEV), torch.from_numpy(beta).to(DEV)
    want = st.copy()
    for t in range(T):
        want = gamma[:, :, t, None, None] * want          # float32 products, frame by frame
    for state in ("given", None, "in_place"):
        s_in = None if state is None else torch.from_numpy(st).to(DEV)
        kw = {"state_out": s_in} if state == "in_place" else {}
        out, so = F.frame_fwd(qkv, qkv, qkv, g_t, b_t, s_in, **kw)
        torch.cuda.synchronize()
        assert out.shape == (B, H, T, S, D) and so.shape == (B, H, D, D)
        if B * H == 0:
            continue
        ref = want if state is not None else np.zeros_like(st)
        assert torch.equal(so.cpu(), torch.from_numpy(ref)), state
        if state is None:
            continue
        for b in range(B):
            for h in range(H):
                e = np.zeros((T, S, D))
                _, M = oracle.gdn_head(e, e, e, gamma[b, h], beta[b, h], st[b, h])
                assert rel_l2(_to_np(so[b, h]), M) <= 1e-6
    # the key-scale entry point takes the same route
    if B * H > 0:
        _, so = F.frame_fwd(qkv, qkv, qkv, g_t, b_t, torch.from_numpy(st).to(DEV), key_scale=0.25)
        torch.cuda.synchronize()
        assert torch.equal(so.cpu(), torch.from_numpy(want))


def test_fused_kernel_wait_failure_ends_without_hang():
    """With a one-poll wait limit the fused kernel's waits run out on
    purpose: the kernel still ends, every row of state_out and every frame
    of out is either exact or NaN (and some are NaN), gdn_fused_status
    reports the timeout, and the next call, with the default limit, starts
    from a fresh control block, is exact again and reports success."""
    import ctypes
    from frame_wise_gated_fwd_amd._lib import Shape
    w = Workload(name="fused_fail", B=1, H=16, T=100, S=64, D=128, in_dtype="bf16", seed=61,
                 gamma_range=(0.95, 1.0), beta_kind="sigmoid_normal", state_std=0.02)
    L = F.lib()
    shp = Shape(w.B, w.H, w.T, w.S, w.D)
    assert L.gdn_path(ctypes.byref(shp), 1) == 2
    x = device_inputs(w, DEV)
    args = (x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    ws = torch.empty(L.gdn_workspace_bytes(ctypes.byref(shp), 1), dtype=torch.uint8, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws_ptr = ctypes.c_void_p(ws.data_ptr())
    ref_out, ref_st = F.frame_fwd(*args, workspace=ws)
    assert L.gdn_fused_status(ws_ptr, stream) == 0
    log("  one-poll waits")
    prev = L.gdn_set_spin_limit(1)
    try:
        out, st = F.frame_fwd(*args, workspace=ws)
        status = L.gdn_fused_status(ws_ptr, stream)
    finally:
        L.gdn_set_spin_limit(prev)
    assert status == 9, status  # GDN_E_TIMEOUT
    nan_rows = torch.isnan(st).all(dim=-1)
    exact_rows = (st == ref_st).all(dim=-1)
    nan_frames = torch.isnan(out).flatten(3).all(dim=-1)
    exact_frames = (out == ref_out).flatten(3).all(dim=-1)
    log(f"  rows given up: {int(nan_rows.sum())} of {nan_rows.numel()}; "
        f"frames given up: {int(nan_frames.sum())} of {nan_frames.numel()}")
    assert bool((nan_rows | exact_rows).all())
    assert bool(nan_rows.any())
    assert bool((nan_frames | exact_frames).all())
    assert bool(nan_frames.any())
    out2, st2 = F.frame_fwd(*args, workspace=ws)
    assert L.gdn_fused_status(ws_ptr, stream) == 0
    assert torch.equal(out2, ref_out) and torch.equal(st2, ref_st)


def test_fused_kernel_completes_beside_other_work():
    """The fused kernel is launched the ordinary way, with no guarantee that
    all its workgroups are resident at once: roles go by start order, so it
    must make progress while another stream holds compute units and its
    workgroups start piecemeal.  Large copies run on a side stream while
    fused calls are launched on the main one; every call must equal the call
    made alone, bit for bit, and report success."""
    import ctypes
    from frame_wise_gated_fwd_amd._lib import Shape
    w = CLIP_5S.with_(T=100, S=300, name="clip_t100_s300_busy", state_std=0.02)
    L = F.lib()
    shp = Shape(w.B, w.H, w.T, w.S, w.D)
    assert L.gdn_path(ctypes.byref(shp), 1) == 2
    x = device_inputs(w, DEV)
    args = (x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    ws = torch.empty(L.gdn_workspace_bytes(ctypes.byref(shp), 1), dtype=torch.uint8, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws_ptr = ctypes.c_void_p(ws.data_ptr())
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    ref_out, ref_st = F.frame_fwd(*args, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    alone = e0.elapsed_time(e1)
    src = torch.empty(1 << 29, dtype=torch.float32, device=DEV).fill_(1.0)  # 2 GiB
    dst = torch.empty_like(src)
    side = torch.cuda.Stream()
    for rnd in range(3):
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for _ in range(3):
                dst.copy_(src)
        e0.record()
        out, st = F.frame_fwd(*args, workspace=ws)
        e1.record()
        status = L.gdn_fused_status(ws_ptr, stream)
        torch.cuda.synchronize()
        # a longer call than alone means the copies held compute units meanwhile
        log(f"  round {rnd}: status {status}, {e0.elapsed_time(e1):.3f} ms beside the copies, {alone:.3f} ms alone")
        assert status == 0
        assert torch.equal(out, ref_out) and torch.equal(st, ref_st)
    del src, dst
    torch.cuda.empty_cache()


def test_fused_calls_on_many_streams():
    """Fused calls issued on six streams at once, each with its own
    workspace and output: the library runs fused launches of one device one
    after another (each holds up to 16 state-pass workgroups per XCD while it
    waits for workers), so all of them finish, equal the call made alone bit
    for bit, and report success."""
    import ctypes
    from frame_wise_gated_fwd_amd._lib import Shape
    w = CLIP_5S.with_(T=40, S=200, name="clip_t40_s200_streams", state_std=0.02)
    L = F.lib()
    shp = Shape(w.B, w.H, w.T, w.S, w.D)
    assert L.gdn_path(ctypes.byref(shp), 1) == 2
    x = device_inputs(w, DEV)
    args = (x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    ref_out, ref_st = F.frame_fwd(*args)
    torch.cuda.synchronize()
    n = 6
    streams = [torch.cuda.Stream() for _ in range(n)]
    wsb = L.gdn_workspace_bytes(ctypes.byref(shp), 1)
    wss = [torch.empty(wsb, dtype=torch.uint8, device=DEV) for _ in range(n)]
    outs = [torch.empty_like(ref_out) for _ in range(n)]
    sts = [torch.empty_like(ref_st) for _ in range(n)]
    for rnd in range(2):
        for i in range(n):
            outs[i].fill_(float("nan"))
        torch.cuda.synchronize()
        for i in range(n):
            with torch.cuda.stream(streams[i]):
                F.frame_fwd(*args, out=outs[i], state_out=sts[i], workspace=wss[i])
        torch.cuda.synchronize()
        for i in range(n):
            status = L.gdn_fused_status(ctypes.c_void_p(wss[i].data_ptr()), ctypes.c_void_p(streams[i].cuda_stream))
            assert status == 0, (rnd, i, status)
            assert torch.equal(outs[i], ref_out) and torch.equal(sts[i], ref_st), (rnd, i)
        log(f"  round {rnd}: {n} streams exact")


def test_fused_kernel_long_sequence():
    """4,000 frames, four times the 60 s workload's chain: the fused kernel's
    rings wrap 125 times and the state carries through 4,000 dependent steps;
    output on sampled frames and the whole final state against the oracle."""
    w = Workload(name="long4000", B=1, H=2, T=4000, S=40, D=128, in_dtype="bf16", seed=63,
                 gamma_range=(0.99, 1.0), beta_kind="sigmoid_normal", state_std=0.02)
    _forward_parity(w, frames=sample_frames(w.T, seed=6))
