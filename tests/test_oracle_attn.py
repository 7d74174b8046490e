"""Pins for the fp64 oracle of the softmax attention block with attention
sinks and local temporal windows (oracle/attn_ref.py).  Each pin ties the
oracle to something outside it:

* visibility: which key frames a query frame sees, against tables worked by
  hand (tests/golden/attn_visibility.json) -- and not through the oracle's own
  helper but by perturbing one key frame at a time and watching which query
  frames' outputs move;
* the arithmetic: torch's scaled_dot_product_attention (float64, CPU) with
  the hand tables' mask expanded to tokens, and torch.logsumexp for the lse;
* worked examples with their numbers derived by hand
  (tests/golden/attn_hand.json);
* closed forms: zero queries give the mean of the visible values and
  lse = ln(number of visible keys); a lone visible key gives its value.

Planted mistakes (copies of the oracle with one plausible error) must each be
caught by one of these pins.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle.attn_ref import Layout, attn_head, attn_frame
from oracle import as_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _visibility_cases():
    with open(os.path.join(GOLDEN, "attn_visibility.json")) as f:
        cases = json.load(f)["cases"]
    return [(Layout(**c["layout"]), c["T"], {int(t): v for t, v in c["visible"].items()}) for c in cases]


def _rand(T, S, D, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [rng.standard_normal((T, S, D)) for _ in range(3)]


# -- the pins, each a function of an implementation with attn_head's signature --
def pin_visibility(impl):
    """Perturb the keys and values of one frame u at a time: exactly the query
    frames that see u (by the hand tables) may change."""
    for i, (lay, T, vis) in enumerate(_visibility_cases()):
        q, k, v = _rand(T, 2, 3, 100 + i)
        O, _ = impl(q, k, v, lay)
        for u in range(T):
            k2, v2 = k.copy(), v.copy()
            k2[u] += 0.7
            v2[u] -= 1.3
            O2, _ = impl(q, k2, v2, lay)
            moved = {t for t in range(T) if not np.allclose(O2[t], O[t], rtol=0, atol=1e-13)}
            want = {t for t, fr in vis.items() if u in fr}
            checked = set(vis)  # frames the table lists
            if moved & checked != want:
                return False, f"layout {lay}: perturbing frame {u} moved {sorted(moved & checked)}, want {sorted(want)}"
    return True, ""


def _token_mask(vis, T, S):
    frame_ok = np.zeros((T, T), dtype=bool)
    for t, fr in vis.items():
        frame_ok[t, fr] = True
    return np.kron(frame_ok, np.ones((S, S), dtype=bool))


def pin_library(impl):
    """torch's scaled_dot_product_attention and logsumexp (float64) with the
    hand tables' masks, on the frames the tables list completely."""
    for i, (lay, T, vis) in enumerate(_visibility_cases()):
        if len(vis) != T:
            continue
        S, D = 3, 5
        q, k, v = _rand(T, S, D, 200 + i)
        O, lse = impl(q, k, v, lay)
        mask = torch.from_numpy(_token_mask(vis, T, S))
        tq, tk, tv = (torch.from_numpy(a.reshape(T * S, D)) for a in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=mask[None])[0]
        scores = (tq @ tk.T) * D ** -0.5
        ref_lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=1)
        if not np.allclose(O.reshape(T * S, D), ref.numpy(), rtol=1e-12, atol=1e-12):
            return False, f"O differs from torch for layout {lay}"
        if not np.allclose(lse.reshape(T * S), ref_lse.numpy(), rtol=1e-12, atol=1e-12):
            return False, f"lse differs from torch for layout {lay}"
    return True, ""


def pin_hand(impl):
    with open(os.path.join(GOLDEN, "attn_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v = (np.array(c[n], dtype=np.float64) for n in ("q", "k", "v"))
        O, lse = impl(q, k, v, Layout(**c["layout"]))
        if not (np.allclose(O, np.array(c["O"]), rtol=1e-14, atol=1e-14)
                and np.allclose(lse, np.array(c["lse"]), rtol=1e-14, atol=1e-14)):
            return False, c["what"][:60]
    return True, ""


def pin_closed_forms(impl):
    lay, T = Layout(sink=1, first_chunk=1, chunk=2, window=2), 7
    S, D = 3, 4
    _, k, v = _rand(T, S, D, 300)
    O, lse = impl(np.zeros((T, S, D)), k, v, lay)
    vis = {0: [0], 1: [0, 1, 2], 2: [0, 1, 2], 3: [0, 1, 2, 3, 4], 4: [0, 1, 2, 3, 4], 5: [0, 3, 4, 5, 6],
           6: [0, 3, 4, 5, 6]}  # chunks 0:{0} 1:{1,2} 2:{3,4} 3:{5,6}, worked by hand
    for t, fr in vis.items():
        mean = np.concatenate([v[u] for u in fr]).mean(axis=0)
        if not np.allclose(O[t], mean, rtol=1e-13, atol=1e-13):
            return False, f"zero queries: frame {t} is not the mean of its visible values"
        if not np.allclose(lse[t], np.log(len(fr) * S), rtol=1e-13, atol=1e-13):
            return False, f"zero queries: lse of frame {t}"
    # one frame of one token: the lone key's value, lse = its score
    q, k, v = _rand(1, 1, 6, 301)
    O, lse = impl(q, k, v, Layout(sink=0, first_chunk=1, chunk=1, window=1))
    if not (np.allclose(O, v, rtol=1e-14, atol=0) and np.allclose(lse[0, 0], q[0, 0] @ k[0, 0] / np.sqrt(6))):
        return False, "a lone key must give its value"
    return True, ""


PINS = {"visibility": pin_visibility, "library": pin_library, "hand": pin_hand, "closed_forms": pin_closed_forms}


@pytest.mark.parametrize("name", sorted(PINS))
def test_attention_oracle_pin(name):
    ok, detail = PINS[name](attn_head)
    assert ok, detail


def test_visible_frames_helper_matches_hand_tables():
    for lay, T, vis in _visibility_cases():
        for t, fr in vis.items():
            assert lay.visible_frames(t, T) == fr, (lay, t)


def test_out_frames_subset_equals_full_rows():
    lay, T = Layout(sink=1, first_chunk=1, chunk=2, window=2), 7
    q, k, v = _rand(T, 3, 4, 400)
    O, lse = attn_head(q, k, v, lay)
    F = [6, 0, 3, 3]
    Os, lses = attn_head(q, k, v, lay, out_frames=F)
    assert np.array_equal(Os, O[F]) and np.array_equal(lses, lse[F])
    with pytest.raises(ValueError):
        attn_head(q, k, v, lay, out_frames=[7])


# -- planted mistakes -----------------------------------------------------------
def _copy(visible=None, scale=None, frame_fn=None):
    """attn_head with one part replaced."""
    def impl(q, k, v, layout, out_frames=None):
        q, k, v = as_f64(q), as_f64(k), as_f64(v)
        T, S, D = q.shape
        vis = visible or (lambda lay, t: lay.visible_frames(t, T))
        O = np.empty_like(q)
        lse = np.empty((T, S))
        for t in range(T):
            fr = vis(layout, t)
            if frame_fn:
                O[t], lse[t] = frame_fn(q[t], k, v, fr)
                continue
            K = np.concatenate([k[u] for u in fr])
            V = np.concatenate([v[u] for u in fr])
            s = (q[t] @ K.T) * (scale(D) if scale else 1 / np.sqrt(D))
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            O[t], lse[t] = (e / z) @ V, (m + np.log(z))[:, 0]
        return O, lse
    return impl


def _vis_rule(kind):
    def vis(lay, t):
        T = 64  # enough frames for every test layout; _trim cuts to the head's T
        c = lay.chunk_of(t)
        lo = max(0, c - lay.window + 1)
        out = []
        for u in range(T):
            cu = lay.chunk_of(u)
            if kind == "window_one_more":      # one chunk too many in the window
                ok = cu <= c and (u < lay.sink or cu >= max(0, lo - 1))
            elif kind == "no_sink":
                ok = lo <= cu <= c
            elif kind == "causal_inside_chunk":  # a frame does not see later frames of its own chunk
                ok = cu <= c and (u < lay.sink or cu >= lo) and u <= t
            elif kind == "future_sink":          # sinks visible even from earlier chunks
                ok = u < lay.sink or lo <= cu <= c
            elif kind == "frames_not_chunks":    # the window counted in frames, not chunks
                ok = u <= t and (u < lay.sink or u > t - lay.window)
            else:
                raise ValueError(kind)
            out.append(ok)
        return [u for u, ok in enumerate(out) if ok]
    return vis


def _trim(vis):
    # restrict a rule written for up to 64 frames to the head's T frames
    def impl(q, k, v, layout, out_frames=None):
        T = q.shape[0]
        return _copy(visible=lambda lay, t: [u for u in vis(lay, t) if u < T])(q, k, v, layout)
    return impl


def _lse_without_max(q_t, k, v, fr):
    K = np.concatenate([k[u] for u in fr])
    V = np.concatenate([v[u] for u in fr])
    s = q_t @ K.T / np.sqrt(q_t.shape[1])
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ V, np.log(z)[:, 0]


def _softmax_over_queries(q_t, k, v, fr):
    K = np.concatenate([k[u] for u in fr])
    V = np.concatenate([v[u] for u in fr])
    s = q_t @ K.T / np.sqrt(q_t.shape[1])
    e = np.exp(s - s.max(axis=0, keepdims=True))
    p = e / e.sum(axis=0, keepdims=True)
    return p @ V, np.log(np.exp(s).sum(axis=1))


def _values_of_queries(q_t, k, v, fr):
    O, lse = attn_frame(q_t, k, v, fr)
    K = np.concatenate([k[u] for u in fr])
    s = q_t @ K.T / np.sqrt(q_t.shape[1])
    p = np.exp(s - lse[:, None])
    return p @ K, lse  # weights applied to the keys instead of the values


MUTANTS = {
    "no_scale": _copy(scale=lambda D: 1.0),
    "scale_1_over_D": _copy(scale=lambda D: 1.0 / D),
    "window_one_more": _trim(_vis_rule("window_one_more")),
    "no_sink": _trim(_vis_rule("no_sink")),
    "causal_inside_chunk": _trim(_vis_rule("causal_inside_chunk")),
    "future_sink": _trim(_vis_rule("future_sink")),
    "frames_not_chunks": _trim(_vis_rule("frames_not_chunks")),
    "lse_without_max": _copy(frame_fn=_lse_without_max),
    "softmax_over_queries": _copy(frame_fn=_softmax_over_queries),
    "weights_on_keys": _copy(frame_fn=_values_of_queries),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_attention_pins_catch_mutant(name):
    with np.errstate(all="ignore"):
        results = {p: fn(MUTANTS[name])[0] for p, fn in PINS.items()}
    assert not all(results.values()), f"mutant {name} passed every pin"
