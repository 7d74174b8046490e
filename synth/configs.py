"""Seeded synthetic workloads for the frame-wise Gated DeltaNet forward.

The SANA-WM pages measure on their own unreleased model and data, so every
workload here is synthetic.  The shapes follow the pages' long-video setting:
a 60 s, 16 fps, 720p clip is 961 latent frames ("SANA-WM: NVIDIA puts a
one-minute world model on a single GPU", section "why one minute is hard";
bilibili cv49203711, third key point).  Heads H=16, head dim D=128 and a 22x40
token grid per latent frame (S=880) are the workload sizes this library is
measured on; the pages state neither S nor the GDN head dim.

This module holds only shapes and value distributions.  It contains none of
the recurrence's arithmetic and is shared by the GPU tests and the oracle
tests as the single source of seeded inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    S: int
    D: int
    in_dtype: str                      # "f32" or "bf16"
    seed: int
    gamma_range: Tuple[float, float]   # gamma_t ~ U(lo, hi), one per (b,h,t)
    beta_kind: str                     # "sigmoid_normal" or "uniform"
    beta_range: Tuple[float, float] = (0.0, 1.0)   # used when beta_kind == "uniform"
    state_std: Optional[float] = None  # None -> zero initial state; else N(0, std) fp32
    boost_frac: float = 0.0            # fraction of token rows per frame with boosted keys
    boost_mult: float = 1.0            # multiplier for those rows (before key scaling)
    # streaming partition (frames per successive call); empty -> one call
    stream_chunks: Tuple[int, ...] = field(default_factory=tuple)
    tol: float = 2e-3                  # relative L2 tolerance for O and the final state
    keys_prescaled: bool = True        # False: raw keys, the library applies key_scale itself

    @property
    def heads(self) -> int:
        return self.B * self.H

    @property
    def key_scale(self) -> float:
        """1/sqrt(D*S): keys are pre-scaled by it before they reach the library,
        unless keys_prescaled is False (then the caller passes it as key_scale)."""
        return 1.0 / (self.D * self.S) ** 0.5

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def _stream_partition(T: int, chunk: int) -> Tuple[int, ...]:
    full, rest = divmod(T, chunk)
    return tuple([chunk] * full + ([rest] if rest else []))


TINY_F32 = Workload(
    name="tiny_f32", B=1, H=2, T=8, S=16, D=32, in_dtype="f32", seed=1,
    gamma_range=(0.9, 1.0), beta_kind="sigmoid_normal", tol=1e-5)

CLIP_5S = Workload(
    name="clip5s_bf16", B=1, H=16, T=81, S=880, D=128, in_dtype="bf16", seed=2,
    gamma_range=(0.95, 1.0), beta_kind="sigmoid_normal")

SEQ_60S = Workload(
    name="seq60s_720p_bf16", B=1, H=16, T=961, S=880, D=128, in_dtype="bf16", seed=3,
    gamma_range=(0.95, 1.0), beta_kind="sigmoid_normal", state_std=0.02)

# Same tensors as SEQ_60S, processed as 24 calls of 40 frames plus a final
# 1-frame call, carrying the fp32 state between calls.
STREAM_60S = SEQ_60S.with_(name="stream60s_bf16", stream_chunks=_stream_partition(961, 40))

STRESS_B4 = Workload(
    name="stress_b4_bf16", B=4, H=16, T=961, S=880, D=128, in_dtype="bf16", seed=5,
    gamma_range=(0.999, 1.0), beta_kind="uniform", beta_range=(0.9, 1.0),
    boost_frac=0.1, boost_mult=4.0)

WORKLOADS = {w.name: w for w in (TINY_F32, CLIP_5S, SEQ_60S, STREAM_60S, STRESS_B4)}


@dataclass(frozen=True)
class AttnWorkload:
    """A softmax attention block with attention sinks and a local temporal
    window over the same token layout as the GDN block ([B, H, T, S, D]).
    The pages name sinks and windows for the chunk-causal variant but give
    no sizes; sink, first_chunk, chunk and window are this workload's
    choice (frames of sink, frames of chunk 0, frames per later chunk,
    chunks per window)."""
    name: str
    B: int
    H: int
    T: int
    S: int
    D: int
    seed: int
    sink: int
    first_chunk: int
    chunk: int
    window: int
    tol: float = 2e-3

    def with_(self, **kw) -> "AttnWorkload":
        d = dict(self.__dict__)
        d.update(kw)
        return AttnWorkload(**d)


# The 60 s sequence's token layout: the clip's first latent frame alone as
# chunk 0 and as the attention sink, then chunks of 4 latent frames (a
# quarter second at 16 latent frames per second), each query seeing its own
# chunk and the one before it: at most 1 + 8 frames = 7,920 keys.
ATTN_60S = AttnWorkload(name="attn60s_sink1_chunk4_win2_bf16", B=1, H=16, T=961, S=880, D=128, seed=7,
                        sink=1, first_chunk=1, chunk=4, window=2)
ATTN_WORKLOADS = {ATTN_60S.name: ATTN_60S}

# The workload the throughput figure is quoted on (one GPU's share of the
# 60 s, 720p sequence).
BENCH_WORKLOAD = SEQ_60S
