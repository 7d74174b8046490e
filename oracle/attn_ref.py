"""Plain, slow fp64 CPU oracle for the softmax attention block of the
chunk-causal variant: attention-sink frames plus a local temporal window.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or run anything in this directory.
The GPU library never calls it, and it imports nothing from the GPU package.

What the pages say ("SANA-WM: NVIDIA puts a one-minute world model on a
single GPU", zhichai.net):
  * section "1. Hybrid Linear Attention -- Gated DeltaNet + Softmax": 5 of
    the 20 blocks (layers 3, 7, 11, 15, 19) are softmax attention blocks,
    which carry exact long-range recall next to the frame-wise GDN blocks;
  * training pipeline, Stage 4: for the chunk-causal autoregressive variant
    the softmax layers get attention-sink tokens and local temporal windows,
    so that memory stays constant over a long rollout.
The pages give no sink count, window length or chunk size; the readings
taken here (every one a parameter of the layout below):
  * the token sequence of one head is T latent frames of S tokens;
  * frames are grouped into generation chunks: chunk 0 holds the first
    `first_chunk` frames, every later chunk `chunk` frames;
  * a query token of chunk c sees every token of chunks c - window + 1 .. c
    (the local temporal window, bidirectional inside its own chunk and
    causal across chunks) and every token of the first `sink` frames (the
    attention sinks) that lie in chunks up to c (a sink is never in a
    query's future), and nothing else;
  * the scores are q . k / sqrt(D) and the weights their softmax over the
    visible keys; the output is the weighted sum of the visible values, and
    the log-sum-exp of the scaled scores is returned beside it.

Everything here is float64; bf16 inputs arrive as uint16 bit patterns and
are widened exactly.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .gdn_ref import as_f64


@dataclass(frozen=True)
class Layout:
    """Which key frames a query frame sees (all counts in latent frames)."""
    sink: int          # leading frames (attention sinks) every query of their chunk or later sees
    first_chunk: int   # frames of chunk 0
    chunk: int         # frames of every later chunk
    window: int        # chunks of the local window, the query's own included

    def chunk_of(self, t: int) -> int:
        """Generation chunk holding frame t."""
        return 0 if t < self.first_chunk else 1 + (t - self.first_chunk) // self.chunk

    def visible_frames(self, t: int, T: int) -> List[int]:
        """The key frames a query of frame t attends to, in increasing order:
        the sink frames up to its own chunk, and the frames of its own chunk
        and of the window - 1 chunks before it."""
        c = self.chunk_of(t)
        lo = max(0, c - self.window + 1)
        return [u for u in range(T) if self.chunk_of(u) <= c and (u < self.sink or self.chunk_of(u) >= lo)]


def attn_frame(q_t, k, v, frames: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of the S query tokens of one frame over the tokens of
    `frames`.  q_t: [S, D]; k, v: [T, S, D] (float64).  Returns
    (O_t [S, D], lse_t [S]) with lse the natural log of the sum of the
    exponentials of the scaled scores."""
    D = q_t.shape[1]
    K = np.concatenate([k[u] for u in frames], axis=0)      # [n, D]
    V = np.concatenate([v[u] for u in frames], axis=0)      # [n, D]
    scores = (q_t @ K.T) / np.sqrt(D)                       # [S, n]
    m = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ V, (m + np.log(z))[:, 0]


def attn_head(q, k, v, layout: Layout, out_frames: Optional[Sequence[int]] = None):
    """The attention block of one head.  q, k, v: [T, S, D] (uint16 bf16 bits
    or floats).  Returns (O [F, S, D], lse [F, S]) for the query frames
    out_frames (all frames when None), in that order."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    T = q.shape[0]
    frames = list(range(T)) if out_frames is None else [int(t) for t in out_frames]
    if any(t < 0 or t >= T for t in frames):
        raise ValueError(f"out_frames must lie in 0 .. {T - 1}")
    O = np.empty((len(frames),) + q.shape[1:])
    lse = np.empty((len(frames), q.shape[1]))
    for i, t in enumerate(frames):
        O[i], lse[i] = attn_frame(q[t], k, v, layout.visible_frames(t, T))
    return O, lse


def attn_flops(T: int, S: int, D: int, layout: Layout) -> int:
    """Dense multiply-add count of one head, 2 flops each: Q K^T and P V over
    every visible (query, key) pair."""
    pairs = sum(S * S * len(layout.visible_frames(t, T)) for t in range(T))
    return 4 * pairs * D
