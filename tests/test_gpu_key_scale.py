"""GPU parity of the key scale applied inside the build (gdn_frame_fwd_ks,
gdn_frame_bwd_ks, through the C ABI).

The recurrence runs on ks * K_t, ks = 1/sqrt(D*S) for the pages' setting.
Three kinds of check, on each execution path:
  * raw keys + ks against the fp64 oracle run on ks * K (exact in float64);
  * raw keys scaled by a power of two p, with ks = 1/p, against the plain
    entry point on the original keys: every product and float32 sum scales
    exactly, so the two agree bit for bit;
  * ks = 1 against the plain entry point, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import frame_wise_gated_fwd_amd as F
from synth import Workload, head_inputs
from gpu_util import device_inputs, RelL2, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KEYS = ("dq", "dk", "dv", "dgamma", "dbeta", "dstate")

# path name -> (workload, fused switch); path 2 = fused persistent kernel,
# 1 = three kernels, 0 = the generic kernels.
PATHS = {
    "fused": (Workload(name="ks_fused", B=1, H=2, T=70, S=100, D=128, in_dtype="bf16", seed=91,
                       gamma_range=(0.95, 1.0), beta_kind="sigmoid_normal", state_std=0.02), 2),
    "three_kernel": (Workload(name="ks_3k", B=1, H=3, T=9, S=130, D=128, in_dtype="bf16", seed=92,
                              gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal", state_std=0.02), 1),
    "generic_f32": (Workload(name="ks_f32", B=1, H=2, T=8, S=24, D=48, in_dtype="f32", seed=93,
                             gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal", state_std=0.05,
                             tol=1e-5), 0),
    "generic_bf16_d64": (Workload(name="ks_d64", B=1, H=2, T=6, S=40, D=64, in_dtype="bf16", seed=94,
                                  gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal"), 0),
}


def _to_np(t):
    return t.detach().cpu().float().numpy().astype(np.float64)


def _check_path(w, path):
    from frame_wise_gated_fwd_amd._lib import Shape
    import ctypes
    code = 1 if w.in_dtype == "bf16" else 0
    got = F.lib().gdn_path(ctypes.byref(Shape(w.B, w.H, w.T, w.S, w.D)), code)
    assert got == path, (w.name, got, path)


@pytest.mark.parametrize("name", list(PATHS))
def test_key_scale_forward_against_oracle(name):
    w, path = PATHS[name]
    w = w.with_(keys_prescaled=False)
    _check_path(w, path)
    ks = np.float32(w.key_scale)
    log(f"key scale fwd {name}: T={w.T} S={w.S} D={w.D} {w.in_dtype} ks={float(ks):.6g}")
    x = device_inputs(w, DEV)
    out, st = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"], key_scale=float(ks))
    torch.cuda.synchronize()
    ro, rs = RelL2(), RelL2()
    for b in range(w.B):
        for h in range(w.H):
            d = head_inputs(w, b, h)
            k = oracle.as_f64(d["k"]) * np.float64(ks)      # exact: 8- or 24-bit times 24-bit mantissas
            O, M = oracle.gdn_head(d["q"], k, d["v"], d["gamma"], d["beta"], d["state"])
            ro.add(_to_np(out[b, h]), O)
            rs.add(_to_np(st[b, h]), M)
    log(f"  relL2 O={ro.value:.3e} state={rs.value:.3e} (tol {w.tol:g})")
    assert np.isfinite(ro.value) and ro.value <= w.tol
    assert np.isfinite(rs.value) and rs.value <= w.tol


@pytest.mark.parametrize("name", list(PATHS))
def test_key_scale_power_of_two_is_exact(name):
    """Keys times 64 with ks = 1/64 give the plain call's result bit for bit;
    ks = 1 does too."""
    w, path = PATHS[name]
    _check_path(w, path)
    log(f"key scale exact {name}")
    x = device_inputs(w, DEV)
    ref_out, ref_st = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"])
    k64 = x["k"] * 64                                            # exact in bf16 and f32
    out, st = F.frame_fwd(x["q"], k64, x["v"], x["gamma"], x["beta"], x["state"], key_scale=1.0 / 64)
    one_out, one_st = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"],
                                  key_scale=1.0)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(st, ref_st)
    assert torch.equal(one_out, ref_out) and torch.equal(one_st, ref_st)


def test_key_scale_chunked_matches_single_call():
    """The scale is per call, so a streamed run with it equals one call."""
    w = PATHS["fused"][0].with_(keys_prescaled=False)
    ks = float(np.float32(w.key_scale))
    x = device_inputs(w, DEV)
    out1, st1 = F.frame_fwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["state"], key_scale=ks)
    state = x["state"].clone()
    outs = []
    for t0, t1 in ((0, 66), (66, 70)):                          # fused then three-kernel
        sl = slice(t0, t1)
        o, _ = F.frame_fwd(*(x[n][:, :, sl].contiguous() for n in ("q", "k", "v", "gamma", "beta")),
                           state, state_out=state, key_scale=ks)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=2), out1) and torch.equal(state, st1)


def _bwd_inputs(w, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    d_out = torch.from_numpy(rng.standard_normal((w.B, w.H, w.T, w.S, w.D), dtype=np.float32)).to(torch.bfloat16)
    d_state = rng.standard_normal((w.B, w.H, w.D, w.D), dtype=np.float32) * 0.1
    return d_out, d_state


@pytest.mark.parametrize("T", [7, 65])
def test_key_scale_backward_against_oracle(T):
    """dk is the gradient with respect to the raw keys: ks times the gradient
    with respect to ks * K."""
    w = Workload(name=f"ks_bwd_t{T}", B=1, H=2, T=T, S=90, D=128, in_dtype="bf16", seed=95 + T,
                 gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal", state_std=0.05, keys_prescaled=False)
    ks = np.float32(w.key_scale)
    log(f"key scale bwd T={T}: ks={float(ks):.6g}")
    x = device_inputs(w, DEV)
    d_out, d_state = _bwd_inputs(w, 7 + T)
    got = dict(zip(KEYS, F.frame_bwd(x["q"], x["k"], x["v"], x["gamma"], x["beta"], d_out.to(DEV),
                                     x["state"], torch.from_numpy(d_state).to(DEV), key_scale=float(ks))))
    torch.cuda.synchronize()
    d_out_bits = d_out.view(torch.int16).numpy().view(np.uint16)
    err = {k: RelL2() for k in KEYS}
    for b in range(w.B):
        for h in range(w.H):
            d = head_inputs(w, b, h)
            k = oracle.as_f64(d["k"]) * np.float64(ks)
            ref = oracle.gdn_head_backward(d["q"], k, d["v"], d["gamma"], d["beta"], d["state"],
                                           d_out_bits[b, h], d_state[b, h])
            ref["dk"] = ref["dk"] * np.float64(ks)               # chain rule through ks * K
            for key in KEYS:
                err[key].add(got[key][b, h].cpu().numpy(), ref[key])
    log("  relL2 " + ", ".join(f"{k}={err[k].value:.2e}" for k in KEYS))
    for key in KEYS:
        assert np.isfinite(err[key].value) and err[key].value <= 2e-3, (key, err[key].value)


def test_key_scale_backward_power_of_two_is_exact():
    """Keys times 64 with ks = 1/64: dk is 1/64 of the plain call's dk (both
    are exact power-of-two scalings), every other gradient is equal; ks = 1
    equals the plain call."""
    w = Workload(name="ks_bwd_exact", B=1, H=2, T=66, S=50, D=128, in_dtype="bf16", seed=97,
                 gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal", state_std=0.05)
    x = device_inputs(w, DEV)
    d_out, d_state = _bwd_inputs(w, 11)
    d_out, d_state = d_out.to(DEV), torch.from_numpy(d_state).to(DEV)
    args = (x["q"], x["k"], x["v"], x["gamma"], x["beta"], d_out, x["state"], d_state)
    ref = F.frame_bwd(*args)
    one = F.frame_bwd(*args, key_scale=1.0)
    a64 = list(args)
    a64[1] = x["k"] * 64
    s64 = F.frame_bwd(*a64, key_scale=1.0 / 64)
    torch.cuda.synchronize()
    for key, r, o, s in zip(KEYS, ref, one, s64):
        assert torch.equal(o, r), key
        if key == "dk":
            assert torch.equal(s * 64, r), key
        else:
            assert torch.equal(s, r), key
