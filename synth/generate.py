"""Seeded per-head input generation.

Every head (b, h) of a workload draws its tensors from its own NumPy PCG64
stream seeded with SeedSequence([seed, b, h]), so any head can be regenerated
alone and in any process.  Draw order inside one head's stream:

  1. q  : T*S*D float32 standard normals (frame-major, then token, then dim)
  2. k  : T*S*D float32 standard normals
  3. v  : T*S*D float32 standard normals
  4. gamma : T uniforms on the workload's gamma range (float64, stored float32)
  5. beta  : T draws: standard normal through the logistic function, or a
             uniform on the workload's beta range (float64, stored float32)
  6. boost : for workloads with boosted keys, one permutation of the S token
             rows per frame; the first round(frac*S) rows are boosted
  7. state : D*D float32 normals scaled by state_std, if the workload has one

Keys are multiplied by the boost (exact in float32), then by the key scale
1/sqrt(D*S) in float32 (skipped for workloads whose keys are not
prescaled), and only then rounded to bfloat16 when the workload is bf16.  Rounding is IEEE round-to-nearest-even, which is what
``torch.Tensor.to(torch.bfloat16)`` does.

bf16 tensors are returned as uint16 bit patterns.  This module holds no part
of the recurrence itself.
"""
from __future__ import annotations

import os
from concurrent.futures import ProcessPoolExecutor
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np

from .configs import AttnWorkload, Workload


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.

    NaN inputs are not expected here (all generated values are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def head_rng(w: Workload, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, b, h])))


def head_inputs(w: Workload, b: int, h: int) -> Dict[str, np.ndarray]:
    """Inputs of one head as the library receives them.

    Returns q, k, v with shape [T, S, D] (uint16 bf16 bits or float32),
    gamma, beta with shape [T] float32, and state [D, D] float32 or None."""
    T, S, D = w.T, w.S, w.D
    rng = head_rng(w, b, h)
    n = T * S * D
    q = rng.standard_normal(n, dtype=np.float32).reshape(T, S, D)
    k = rng.standard_normal(n, dtype=np.float32).reshape(T, S, D)
    v = rng.standard_normal(n, dtype=np.float32).reshape(T, S, D)
    gamma = rng.uniform(w.gamma_range[0], w.gamma_range[1], T).astype(np.float32)
    if w.beta_kind == "sigmoid_normal":
        z = rng.standard_normal(T)
        beta = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    elif w.beta_kind == "uniform":
        beta = rng.uniform(w.beta_range[0], w.beta_range[1], T).astype(np.float32)
    else:
        raise ValueError(f"unknown beta_kind {w.beta_kind!r}")
    if w.boost_frac > 0.0:
        nb = int(round(w.boost_frac * S))
        mult = np.float32(w.boost_mult)
        for t in range(T):
            rows = rng.permutation(S)[:nb]
            k[t, rows, :] *= mult
    if w.keys_prescaled:
        k *= np.float32(w.key_scale)
    state = None
    if w.state_std is not None:
        state = (rng.standard_normal(D * D, dtype=np.float32)
                 * np.float32(w.state_std)).reshape(D, D)
    if w.in_dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    elif w.in_dtype != "f32":
        raise ValueError(f"unknown in_dtype {w.in_dtype!r}")
    return {"q": q, "k": k, "v": v, "gamma": gamma, "beta": beta, "state": state}


def attn_head_inputs(w: AttnWorkload, b: int, h: int) -> Dict[str, np.ndarray]:
    """q, k, v of one head of an attention workload: [T, S, D] standard
    normals (float32, drawn q then k then v from SeedSequence([seed, b, h]))
    rounded to bfloat16 bits."""
    T, S, D = w.T, w.S, w.D
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, b, h])))
    n = T * S * D
    out = {}
    for key in ("q", "k", "v"):
        out[key] = f32_to_bf16_bits(rng.standard_normal(n, dtype=np.float32).reshape(T, S, D))
    return out


def _head_job(args):
    w, b, h = args
    return b, h, head_inputs(w, b, h)


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def iter_heads(w: Workload, heads: Optional[Iterable[Tuple[int, int]]] = None,
               workers: Optional[int] = None):
    """Yield (b, h, inputs) for the requested heads, generated in parallel."""
    hs = list(heads) if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    workers = workers or default_workers()
    if workers <= 1 or len(hs) <= 1:
        for b, h in hs:
            yield b, h, head_inputs(w, b, h)
        return
    with ProcessPoolExecutor(max_workers=min(workers, len(hs))) as ex:
        for res in ex.map(_head_job, [(w, b, h) for b, h in hs]):
            yield res


def full_inputs(w: Workload, workers: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All heads stacked: q/k/v [B,H,T,S,D], gamma/beta [B,H,T], state [B,H,D,D] or None."""
    B, H, T, S, D = w.B, w.H, w.T, w.S, w.D
    qdt = np.uint16 if w.in_dtype == "bf16" else np.float32
    out = {
        "q": np.empty((B, H, T, S, D), qdt),
        "k": np.empty((B, H, T, S, D), qdt),
        "v": np.empty((B, H, T, S, D), qdt),
        "gamma": np.empty((B, H, T), np.float32),
        "beta": np.empty((B, H, T), np.float32),
        "state": None if w.state_std is None else np.empty((B, H, D, D), np.float32),
    }
    for b, h, d in iter_heads(w, workers=workers):
        for key in ("q", "k", "v", "gamma", "beta"):
            out[key][b, h] = d[key]
        if out["state"] is not None:
            out["state"][b, h] = d["state"]
    return out


def head_list(w: Workload) -> List[Tuple[int, int]]:
    return [(b, h) for b in range(w.B) for h in range(w.H)]
