"""Helpers for the GPU parity tests: seeded inputs to the device, the oracle
run per head in worker processes, and relative-L2 accounting in float64."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ProcessPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from synth import Workload, head_inputs, default_workers


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(w: Workload, dev="cuda:0", heads=None) -> Dict[str, torch.Tensor]:
    """All heads of `w` on the device.  Generation runs per head in worker
    processes and each head is copied to the device as it arrives."""
    B, H, T, S, D = w.B, w.H, w.T, w.S, w.D
    tdt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32
    out = {key: torch.empty((B, H, T, S, D), dtype=tdt, device=dev) for key in ("q", "k", "v")}
    out["gamma"] = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    out["beta"] = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    out["state"] = (None if w.state_std is None
                    else torch.empty((B, H, D, D), dtype=torch.float32, device=dev))
    hs = [(b, h) for b in range(B) for h in range(H)]
    workers = min(default_workers(), len(hs))
    def put(b, h, d):
        for key in ("q", "k", "v"):
            a = d[key]
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
                else torch.from_numpy(a)
            out[key][b, h].copy_(t)
        out["gamma"][b, h].copy_(torch.from_numpy(d["gamma"]))
        out["beta"][b, h].copy_(torch.from_numpy(d["beta"]))
        if out["state"] is not None:
            out["state"][b, h].copy_(torch.from_numpy(d["state"]))
    if workers <= 1:
        for b, h in hs:
            put(b, h, head_inputs(w, b, h))
    else:
        with ProcessPoolExecutor(max_workers=workers) as ex:
            futs = {ex.submit(head_inputs, w, b, h): (b, h) for b, h in hs}
            for fut, (b, h) in futs.items():
                put(b, h, fut.result())
    torch.cuda.synchronize()
    return out


def _oracle_job(args):
    w, b, h, frames = args
    from threadpoolctl import threadpool_limits
    import oracle
    with threadpool_limits(1):
        d = head_inputs(w, b, h)
        O, M = oracle.gdn_head(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["state"],
                               out_frames=frames)
    return b, h, O, M


def oracle_heads(w: Workload, heads: Sequence[Tuple[int, int]], frames: Optional[Sequence[int]] = None,
                 workers: Optional[int] = None):
    """Yield (b, h, O [len(frames) or T, S, D] f64, M_T [D, D] f64) per head."""
    workers = workers or min(default_workers(), len(heads))
    jobs = [(w, b, h, None if frames is None else list(frames)) for b, h in heads]
    if workers <= 1:
        for j in jobs:
            yield _oracle_job(j)
        return
    with ProcessPoolExecutor(max_workers=workers) as ex:
        for res in ex.map(_oracle_job, jobs):
            yield res


class RelL2:
    """sqrt(sum (x - ref)^2) / sqrt(sum ref^2), accumulated in float64."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0
        self.max_abs = 0.0

    def add(self, x, ref) -> None:
        x = np.asarray(x, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        d = x - ref
        self.num += float(np.sum(d * d))
        self.den += float(np.sum(ref * ref))
        if d.size:
            self.max_abs = max(self.max_abs, float(np.max(np.abs(d))))

    @property
    def value(self) -> float:
        return float(np.sqrt(self.num / self.den)) if self.den > 0 else float(np.sqrt(self.num))


def rel_l2(x, ref) -> float:
    r = RelL2()
    r.add(x, ref)
    return r.value


def sample_frames(T: int, seed: int = 0, extra: int = 6) -> List[int]:
    base = {0, 1, min(2, T - 1), T // 4, T // 2, (3 * T) // 4, max(T - 3, 0), max(T - 2, 0), T - 1}
    rng = np.random.Generator(np.random.PCG64(seed))
    base.update(int(x) for x in rng.integers(0, T, size=extra))
    return sorted(base)
