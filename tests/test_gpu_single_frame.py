"""The single-frame kernels (T == 1, bf16, D == 128: the call of frame-by-frame
generation) through the C ABI: against the fp64 oracle at float32-grade
tolerance (relative L2 <= 1e-5 for the output and the state, every head and
frame on its own), against the three-kernel path (the same step with the
frame's tokens summed in another order), over many calls in a row, and on
their edge cases: head counts that are not a multiple of 8, one
token, more token tiles than waves, a zero state, the state updated in
place, bf16 output, the key scale and gates from activations, and sizes
whose byte offsets pass 2^31 (many heads; one very long frame)."""
import ctypes
import math

import pytest
import torch

import frame_wise_gated_fwd_amd as F
from frame_wise_gated_fwd_amd._lib import Shape, GDN_BF16, GDN_F32, GDN_PATH_FRAME, GDN_PATH_MFMA
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


def _raw_frame_call(x, out, state_out, ws):
    """gdn_frame_fwd through the C ABI with an explicit workspace (None: no
    workspace, so the single-frame kernel runs one workgroup per row block)."""
    B, H, _, S, D = x["q"].shape
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = F.lib().gdn_frame_fwd(ctypes.byref(Shape(B, H, 1, S, D)), GDN_BF16, GDN_F32, P(x["q"]), P(x["k"]),
                               P(x["v"]), P(x["gamma"]), P(x["beta"]), P(x["state"]), P(out), P(state_out),
                               P(ws), 0 if ws is None else ws.numel(), st)
    assert rc == 0, f"gdn_frame_fwd returned {rc}"


def _split_ws(x):
    B, H, _, S, D = x["q"].shape
    n = F.lib().gdn_workspace_bytes(ctypes.byref(Shape(B, H, 1, S, D)), GDN_BF16)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=DEV), n


@pytest.mark.parametrize("H,S", [(16, 880), (3, 100), (1, 64), (16, 17)], ids=lambda v: str(v))
def test_single_frame_split_and_one_workgroup_forms(H, S):
    """Up to 16 heads, with the workspace the query asks for, a row block's
    even and odd token tiles go to two workgroups that swap their partial
    sums; without a workspace one workgroup sums all of them.  Both forms
    against the oracle at float32-grade tolerance, and against each other
    (they add the same products in another order).  S = 64 and 17: one tile,
    so the odd half of every pair has no tokens."""
    w = CLIP_5S.with_(T=1, H=H, S=S, name=f"frame1_split_{H}_{S}", state_std=0.05, seed=400 + H + S)
    x = device_inputs(w, DEV)
    ws, n = _split_ws(x)
    assert n > 0
    o_split = torch.empty(x["q"].shape, dtype=torch.float32, device=DEV)
    s_split = torch.empty(x["state"].shape, dtype=torch.float32, device=DEV)
    o_one, s_one = torch.empty_like(o_split), torch.empty_like(s_split)
    _raw_frame_call(x, o_split, s_split, ws)
    _raw_frame_call(x, o_one, s_one, None)
    torch.cuda.synchronize()
    worst = 0.0
    for h in range(H):
        for o, st in ((o_split, s_split), (o_one, s_one)):
            ro, rs = _oracle_head(x, o, st, 0, h)
            worst = max(worst, ro, rs)
    ro, rs = _rel(o_split, o_one), _rel(s_split, s_one)
    log(f"  split vs one workgroup: relL2 O={ro:.3e} state={rs:.3e}; worst against the oracle {worst:.3e}")
    assert worst <= TOL
    assert ro <= 1e-6 and rs <= 1e-6
    assert torch.isfinite(o_split).all() and torch.isfinite(s_split).all()


def test_single_frame_split_in_place_over_many_calls():
    """The split form with state_out == state_in: the workgroup that writes a
    pair's rows is the second of the pair to finish its sums, after both have
    read them.  20 calls in a row in place equal 20 calls alternating two
    state buffers, bit for bit, on fresh inputs each call."""
    w = CLIP_5S.with_(T=20, H=16, S=880, name="frame1_split_inplace", state_std=0.05, seed=431)
    x = device_inputs(w, DEV)
    ws, _ = _split_ws({"q": x["q"][:, :, :1]})
    st_in = x["state"].clone()
    bufs = [x["state"].clone(), torch.empty_like(x["state"])]
    o_a = torch.empty((w.B, w.H, 1, w.S, w.D), dtype=torch.float32, device=DEV)
    o_b = torch.empty_like(o_a)
    for t in range(w.T):
        f = {k: x[k][:, :, t:t + 1].contiguous() for k in ("q", "k", "v", "gamma", "beta")}
        _raw_frame_call(dict(f, state=st_in), o_a, st_in, ws)
        _raw_frame_call(dict(f, state=bufs[t % 2]), o_b, bufs[(t + 1) % 2], ws)
        torch.cuda.synchronize()
        assert torch.equal(o_a, o_b), f"frame {t}: out"
        assert torch.equal(st_in, bufs[(t + 1) % 2]), f"frame {t}: state"
    log(f"  {w.T} in-place split calls equal the two-buffer calls")


def test_single_frame_split_wait_that_runs_out():
    """A tiny spin limit (set from the host) makes the first workgroup of a
    pair give up on its partner almost at once.  Every output value is then
    either the normal result, bit for bit, or NaN (the columns of a
    workgroup that gave up), and the state, which the second of each pair
    writes, is the normal result in place and out of place."""
    w = CLIP_5S.with_(T=1, H=16, S=880, name="frame1_split_giveup", state_std=0.05, seed=433)
    x = device_inputs(w, DEV)
    ws, _ = _split_ws(x)
    o_ref = torch.empty(x["q"].shape, dtype=torch.float32, device=DEV)
    s_ref = torch.empty(x["state"].shape, dtype=torch.float32, device=DEV)
    _raw_frame_call(x, o_ref, s_ref, ws)
    L = F.lib()
    prev = L.gdn_set_spin_limit(1)
    try:
        nan_calls = 0
        for i in range(5):
            o = torch.empty_like(o_ref)
            s = torch.empty_like(s_ref)
            _raw_frame_call(x, o, s, ws)
            st = x["state"].clone()
            o2 = torch.empty_like(o_ref)
            _raw_frame_call(dict(x, state=st), o2, st, ws)
            torch.cuda.synchronize()
            for out in (o, o2):
                nan = torch.isnan(out)
                assert torch.equal(out[~nan], o_ref[~nan]), f"call {i}: a value that is neither NaN nor the result"
                nan_calls += int(nan.any())
            assert torch.equal(s, s_ref) and torch.equal(st, s_ref), f"call {i}: state"
        log(f"  spin limit 1: {nan_calls} of 10 calls had a workgroup give up")
    finally:
        L.gdn_set_spin_limit(prev)
    o = torch.empty_like(o_ref)
    s = torch.empty_like(s_ref)
    _raw_frame_call(x, o, s, ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)


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


# ---------------------------------------------------------------------------
# maximum sizes: byte offsets past 2^31
# ---------------------------------------------------------------------------
def _device_frame(B, H, S, seed):
    """One frame per head, seeded on the device (these sizes are beyond the
    host generators' reach): q, v ~ N(0, 1) and keys N(0, 1) / sqrt(D S),
    all rounded to bf16; gamma ~ U(0.9, 1); beta = sigmoid(N(0, 1)); a
    N(0, 0.05^2) float32 state."""
    D = 128
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = {"q": torch.randn((B, H, 1, S, D), generator=g, device=DEV).to(torch.bfloat16)}
    x["k"] = (torch.randn((B, H, 1, S, D), generator=g, device=DEV) / (D * S) ** 0.5).to(torch.bfloat16)
    x["v"] = torch.randn((B, H, 1, S, D), generator=g, device=DEV).to(torch.bfloat16)
    x["gamma"] = torch.rand((B, H, 1), generator=g, device=DEV) * 0.1 + 0.9
    x["beta"] = torch.sigmoid(torch.randn((B, H, 1), generator=g, device=DEV))
    x["state"] = torch.randn((B, H, D, D), generator=g, device=DEV) * 0.05
    torch.cuda.synchronize()
    return x


def _oracle_head(x, out, st, b, h):
    """The oracle on head (b, h) of the device inputs (bf16 as its bit
    patterns, which the oracle widens exactly); relL2 of the output and the
    state."""
    import oracle
    bits = lambda t: t[b, h].contiguous().view(torch.int16).cpu().numpy().view("uint16")
    f64 = lambda t: t[b, h].double().cpu().numpy()
    O, M = oracle.gdn_head(bits(x["q"]), bits(x["k"]), bits(x["v"]), f64(x["gamma"]), f64(x["beta"]),
                           f64(x["state"]))
    return _rel(out[b, h], torch.from_numpy(O)), _rel(st[b, h], torch.from_numpy(M))


def test_single_frame_many_heads_past_2gib():
    """12288 heads (B = 96, H = 128) of 880 tokens in one call: 2.8 GB per
    input and 5.5 GB of output, so the inputs of heads from 9533 on and the
    output of heads from 4767 on lie beyond 2^31 bytes.  Sampled heads on
    both sides of those lines, and the last, against the oracle."""
    B, H, S = 96, 128, 880
    log(f"single frame, {B * H} heads x {S} tokens")
    assert F.lib().gdn_path(ctypes.byref(Shape(B, H, 1, S, 128)), GDN_BF16) == GDN_PATH_FRAME
    x = _device_frame(B, H, S, seed=11)
    out, st = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    torch.cuda.synchronize()
    for hd in (0, 4766, 4767, 9532, 9533, 12001, B * H - 1):
        b, h = divmod(hd, H)
        ro, rs = _oracle_head(x, out, st, b, h)
        log(f"  head {hd}: relL2 O={ro:.3e} state={rs:.3e}")
        assert ro <= TOL and rs <= TOL


def test_single_frame_long_frame_past_2gib():
    """One head with 4,194,513 tokens (2^22 + 209): 1.07 GB per input, and
    the float32 output of the tokens after the 2^22nd lies beyond 2^31
    bytes; a ragged last tile.  The whole output and the state against the
    oracle.

    Tolerance: each float32 accumulator of the state's sum adds about
    S / 256 products of 32 tokens in sequence (S / 8 tokens per wave, 32
    per MFMA), whose rounding grows like u sqrt(S / 256) (u = 2^-24; 7.6e-6
    here), so the bound is the 880-token one plus four times that.  A wrong
    address past 2^31 bytes would be an O(1) error."""
    S = (1 << 22) + 209
    tol = TOL + 4 * 2.0 ** -24 * math.sqrt(S / 256)
    log(f"single frame, one head x {S} tokens (tol {tol:.2e})")
    x = _device_frame(1, 1, S, seed=12)
    out, st = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    torch.cuda.synchronize()
    ro, rs = _oracle_head(x, out, st, 0, 0)
    log(f"  relL2 O={ro:.3e} state={rs:.3e}")
    assert ro <= tol and rs <= tol
