"""Plain, slow fp64 CPU oracle for the frame-wise Gated DeltaNet forward.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or run anything in this directory.
The GPU library never calls it, and it imports nothing from the GPU package.

What the method computes, from the SANA-WM pages:

* "SANA-WM: NVIDIA puts a one-minute world model on a single GPU"
  (zhichai.net), section "1. Hybrid Linear Attention -- Gated DeltaNet +
  Softmax":
    - a learned decay scalar gamma multiplies the previous recurrent state, so
      stale content fades;
    - a delta-rule strength beta updates only the residual between what the
      state predicts and the target, instead of overwriting the state;
    - the state keeps a constant D x D size however many frames go by;
    - keys are scaled by 1/sqrt(D*S) (D head dim, S spatial tokens per frame),
      which bounds the spectral norm of the transition matrix.
* bilibili cv49203711, fourth key point: the GDN is frame-wise -- one
  recurrent step consumes one whole latent frame rather than one token.
* zhichai.net page, training pipeline, Stage 3: transition matrices compose
  by prefix sums exactly (used by the chunked variant below).

The update this library implements, with state rows indexing value dims and
columns indexing key dims, per head and frame t (K_t, V_t, Q_t are S x D):

    G_t = K_t^T K_t,   U_t = V_t^T K_t
    A_t = gamma_t (I - beta_t G_t)
    M_t = M_{t-1} A_t + beta_t U_t
    O_t = Q_t M_t^T

Readings of points the pages leave open (state orientation, output taken after
the frame's update, gamma not scaling the injection, keys pre-scaled by the
caller, one gamma and one beta per frame) are listed with the design notes.

Everything here is float64.  bf16 inputs arrive as uint16 bit patterns and are
widened exactly, so the oracle sees the same numbers the GPU sees.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


# ----------------------------------------------------------------------------
# input decoding (exact)
# ----------------------------------------------------------------------------
def as_f64(x) -> np.ndarray:
    """Exact widening to float64.  uint16 arrays are bfloat16 bit patterns."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------
# the recurrence, one head
# ----------------------------------------------------------------------------
def frame_maps(k_t: np.ndarray, v_t: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """G_t = K_t^T K_t (key x key) and U_t = V_t^T K_t (value x key) of one frame.

    Both reduce over the S tokens of the frame: one recurrent step sees the
    whole frame (bilibili cv49203711, fourth key point)."""
    return k_t.T @ k_t, v_t.T @ k_t


def transition(g_t: np.ndarray, gamma_t: float, beta_t: float) -> np.ndarray:
    """A_t = gamma_t (I - beta_t G_t): decay of the previous state times the
    delta-rule projection (zhichai.net page, section 1)."""
    d = g_t.shape[0]
    return gamma_t * (np.eye(d) - beta_t * g_t)


def gdn_head(q, k, v, gamma, beta, state=None, keep_states: bool = False, out_frames=None):
    """Frame-wise GDN forward of one head.

    q, k, v: [T, S, D]; gamma, beta: [T]; state: [D, D] or None (zeros).
    Returns (O [T, S, D], M_T [D, D]) and, with keep_states, also the stacked
    states M_1..M_T [T, D, D].  With out_frames (a sequence of frame indices,
    in any order, repeats allowed) row i of O is the output of frame
    out_frames[i], and O is [len(out_frames), S, D]; an index outside
    0 .. T-1 raises ValueError."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    gamma, beta = as_f64(gamma), as_f64(beta)
    T, S, D = q.shape
    M = np.zeros((D, D)) if state is None else as_f64(state).copy()
    wanted = list(range(T)) if out_frames is None else [int(t) for t in out_frames]
    if any(t < 0 or t >= T for t in wanted):
        raise ValueError(f"out_frames must lie in 0 .. {T - 1}")
    rows = {}  # frame -> every position of O that wants it
    for i, t in enumerate(wanted):
        rows.setdefault(t, []).append(i)
    O = np.empty((len(wanted), S, D))
    states = np.empty((T, D, D)) if keep_states else None
    for t in range(T):
        G, U = frame_maps(k[t], v[t])
        M = M @ transition(G, gamma[t], beta[t]) + beta[t] * U
        if t in rows:
            O_t = q[t] @ M.T
            for i in rows[t]:
                O[i] = O_t
        if keep_states:
            states[t] = M
    if keep_states:
        return O, M, states
    return O, M


def gdn_head_residual(q, k, v, gamma, beta, state=None):
    """Same recurrence written as the delta rule literally:
    prediction P = gamma K M^T, residual R = V - P, M <- gamma M + beta R^T K.
    Algebraically identical to gdn_head (expand R^T K); a different operation
    order, used to cross-check it."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    gamma, beta = as_f64(gamma), as_f64(beta)
    T, S, D = q.shape
    M = np.zeros((D, D)) if state is None else as_f64(state).copy()
    O = np.empty((T, S, D))
    for t in range(T):
        R = v[t] - gamma[t] * (k[t] @ M.T)
        M = gamma[t] * M + beta[t] * (R.T @ k[t])
        O[t] = q[t] @ M.T
    return O, M


def build_maps_head(k, v) -> Tuple[np.ndarray, np.ndarray]:
    """Stacked G_t, U_t for every frame of one head: two [T, D, D] arrays."""
    k, v = as_f64(k), as_f64(v)
    T = k.shape[0]
    D = k.shape[2]
    G = np.empty((T, D, D))
    U = np.empty((T, D, D))
    for t in range(T):
        G[t], U[t] = frame_maps(k[t], v[t])
    return G, U


def state_pass_head(G, U, gamma, beta, state=None) -> np.ndarray:
    """M_1..M_T from precomputed G_t, U_t: the sequential state pass alone."""
    G, U = as_f64(G), as_f64(U)
    gamma, beta = as_f64(gamma), as_f64(beta)
    T, D, _ = G.shape
    M = np.zeros((D, D)) if state is None else as_f64(state).copy()
    out = np.empty((T, D, D))
    for t in range(T):
        M = M @ transition(G[t], gamma[t], beta[t]) + beta[t] * U[t]
        out[t] = M
    return out


def output_head(q, states) -> np.ndarray:
    """O_t = Q_t M_t^T for every frame, given the post-update states."""
    q, states = as_f64(q), as_f64(states)
    return np.einsum("tsj,tij->tsi", q, states)


# ----------------------------------------------------------------------------
# affine-map composition (zhichai.net page, training pipeline, Stage 3)
# ----------------------------------------------------------------------------
def compose(first: Tuple[np.ndarray, np.ndarray],
            then: Tuple[np.ndarray, np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Maps f(M) = M A + b.  Applying `first` then `then` gives
    M (A1 A2) + (b1 A2 + b2)."""
    A1, b1 = first
    A2, b2 = then
    return A1 @ A2, b1 @ A2 + b2


def state_pass_chunked(G, U, gamma, beta, state=None, chunk: int = 8) -> np.ndarray:
    """State pass by prefix composition over frame chunks.

    1. inside each chunk, compose the per-frame maps (A_t, b_t) into one map;
    2. fold the chunk maps left to right to get the state entering each chunk;
    3. re-expand each chunk from its entering state.
    Exact up to rounding order; returns M_1..M_T like state_pass_head."""
    G, U = as_f64(G), as_f64(U)
    gamma, beta = as_f64(gamma), as_f64(beta)
    T, D, _ = G.shape
    maps = [(transition(G[t], gamma[t], beta[t]), beta[t] * U[t]) for t in range(T)]
    starts = list(range(0, T, chunk))
    chunk_maps = []
    for s in starts:
        acc = maps[s]
        for t in range(s + 1, min(s + chunk, T)):
            acc = compose(acc, maps[t])
        chunk_maps.append(acc)
    M = np.zeros((D, D)) if state is None else as_f64(state).copy()
    entering = []
    for A, b in chunk_maps:
        entering.append(M)
        M = M @ A + b
    out = np.empty((T, D, D))
    for s, M0 in zip(starts, entering):
        acc = None
        for t in range(s, min(s + chunk, T)):
            acc = maps[t] if acc is None else compose(acc, maps[t])
            out[t] = M0 @ acc[0] + acc[1]
    return out


# ----------------------------------------------------------------------------
# the textbook token-wise gated delta rule (for the S = 1 special case)
# ----------------------------------------------------------------------------
def tokenwise_gated_delta(q, k, v, alpha, beta, state=None):
    """Token-wise gated delta rule over a sequence of single tokens, written
    with vectors and outer products:
        St <- St * alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
        o_t = St q_t.
    q, k, v: [N, D]; alpha, beta: [N]."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    alpha, beta = as_f64(alpha), as_f64(beta)
    N, D = q.shape
    St = np.zeros((D, D)) if state is None else as_f64(state).copy()
    o = np.empty((N, D))
    for n in range(N):
        kk = np.outer(k[n], k[n])
        St = St @ (alpha[n] * (np.eye(D) - beta[n] * kk)) + beta[n] * np.outer(v[n], k[n])
        o[n] = St @ q[n]
    return o, St


# ----------------------------------------------------------------------------
# floating-point operation and byte counts
# ----------------------------------------------------------------------------
def flops_per_head_frame(S: int, D: int) -> int:
    """Dense multiply-add count of one head-frame, 2 flops each:
    K^T K and V^T K (2 S D^2 each), M_{t-1} A_t (2 D^3), Q M^T (2 S D^2)."""
    return 6 * S * D * D + 2 * D ** 3
