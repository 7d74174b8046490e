"""GPU parity of the softmax attention block with attention sinks and a
local temporal window (gdn_attn_fwd) against the fp64 oracle
(oracle/attn_ref.py) on the same seeded inputs.  Tolerance: relative L2
<= 2e-3 (bf16 inputs, float32 accumulation), per frame and per head, for
the output and the log-sum-exp."""
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

import frame_wise_gated_fwd_amd as F
from synth import ATTN_60S, AttnWorkload, attn_head_inputs, default_workers

from gpu_util import log, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _device_inputs(w):
    x = {key: torch.empty((w.B, w.H, w.T, w.S, w.D), dtype=torch.bfloat16, device=DEV) for key in "qkv"}
    for b in range(w.B):
        for h in range(w.H):
            d = attn_head_inputs(w, b, h)
            for key in "qkv":
                x[key][b, h].copy_(torch.from_numpy(d[key].view(np.int16)).view(torch.bfloat16))
    torch.cuda.synchronize()
    return x


def _oracle_job(args):
    w, b, h, frames = args
    from threadpoolctl import threadpool_limits
    from oracle.attn_ref import Layout, attn_head
    with threadpool_limits(1):
        d = attn_head_inputs(w, b, h)
        O, lse = attn_head(d["q"], d["k"], d["v"], Layout(w.sink, w.first_chunk, w.chunk, w.window),
                           out_frames=frames)
    return b, h, O, lse


def _parity(w, frames=None, heads=None):
    log(f"attention {w.name}: B={w.B} H={w.H} T={w.T} S={w.S} sink={w.sink} first={w.first_chunk} "
        f"chunk={w.chunk} window={w.window}")
    x = _device_inputs(w)
    out, lse = F.attn_fwd(x["q"], x["k"], x["v"], w.sink, w.first_chunk, w.chunk, w.window)
    torch.cuda.synchronize()
    hs = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    fr = list(range(w.T)) if frames is None else list(frames)
    jobs = [(w, b, h, fr) for b, h in hs]
    worst_o = worst_l = 0.0
    num = den = 0.0
    with ProcessPoolExecutor(max_workers=min(default_workers(), len(jobs))) as ex:
        for b, h, O, L in ex.map(_oracle_job, jobs):
            og = out[b, h, fr].double().cpu().numpy()
            lg = lse[b, h, fr].double().cpu().numpy()
            num += float(((og - O) ** 2).sum())
            den += float((O ** 2).sum())
            for i in range(len(fr)):
                worst_o = max(worst_o, rel_l2(og[i], O[i]))
                worst_l = max(worst_l, rel_l2(lg[i], L[i]))
    rel = (num / den) ** 0.5
    log(f"  relL2 O={rel:.3e}; worst frame O {worst_o:.3e}, lse {worst_l:.3e} (tol {w.tol:g})")
    assert np.isfinite(rel) and rel <= w.tol
    assert worst_o <= w.tol and worst_l <= w.tol
    return out, lse, x


SMALL = [
    # the hand-worked visibility layouts, ragged token counts (tiles cross frames, key tails of 37 tokens)
    AttnWorkload(name="attn_s1_f1_c3_w2", B=1, H=3, T=10, S=37, D=128, seed=21, sink=1, first_chunk=1, chunk=3,
                 window=2),
    AttnWorkload(name="attn_s2_f2_c2_w1", B=2, H=1, T=7, S=100, D=128, seed=22, sink=2, first_chunk=2, chunk=2,
                 window=1),
    AttnWorkload(name="attn_s0_f1_c1_w3", B=1, H=2, T=6, S=64, D=128, seed=23, sink=0, first_chunk=1, chunk=1,
                 window=3),
    AttnWorkload(name="attn_s3_f1_c4_w2", B=1, H=2, T=14, S=50, D=128, seed=24, sink=3, first_chunk=1, chunk=4,
                 window=2),
    # the 60 s layout on 13 frames of the full 880 tokens (sink frame far from the window at the end)
    ATTN_60S.with_(name="attn60s_t13", H=2, T=13, seed=25),
    # degenerate layouts: one chunk (bidirectional full attention), one token per frame,
    # a window wider than the sequence (pure chunk-causal), a sink wider than the sequence
    AttnWorkload(name="attn_one_chunk", B=1, H=2, T=3, S=90, D=128, seed=26, sink=0, first_chunk=5, chunk=1,
                 window=1),
    AttnWorkload(name="attn_s1_token", B=1, H=2, T=40, S=1, D=128, seed=27, sink=1, first_chunk=1, chunk=4,
                 window=2),
    AttnWorkload(name="attn_wide_window", B=1, H=1, T=9, S=70, D=128, seed=28, sink=0, first_chunk=2, chunk=3,
                 window=100),
    AttnWorkload(name="attn_wide_sink", B=1, H=1, T=9, S=70, D=128, seed=29, sink=50, first_chunk=2, chunk=3,
                 window=1),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_attention_matches_oracle(w):
    _parity(w)


def test_attention_60s_sampled_frames():
    """The full 961-frame, 880-token, 16-head chunk-causal layout: every head
    at 10 frames (the sink chunk, the first chunks, chunk boundaries, the
    end)."""
    frames = [0, 1, 4, 5, 8, 9, 480, 481, 959, 960]
    _parity(ATTN_60S, frames=frames)


def test_attention_is_deterministic_and_lse_optional():
    w = SMALL[0]
    x = _device_inputs(w)
    o1, l1 = F.attn_fwd(x["q"], x["k"], x["v"], w.sink, w.first_chunk, w.chunk, w.window)
    o2, l2 = F.attn_fwd(x["q"], x["k"], x["v"], w.sink, w.first_chunk, w.chunk, w.window, want_lse=False)
    torch.cuda.synchronize()
    assert l2 is None
    assert torch.equal(o1, o2)
