"""Pins for the oracle paths that the full-size GPU parity checks run:

* gdn_head(..., out_frames=F) -- only the requested frames' outputs -- must
  equal rows F of the full output bit for bit, for unsorted and repeated F
  (the full output is pinned by the closed forms, goldens and properties in
  test_oracle_pins.py);
* as_f64 -- the exact bf16 decode the oracle applies to every bf16 input --
  must equal torch's bfloat16 -> float64 widening on every one of the 65,536
  bit patterns.

Each pin is also run on planted mistakes (copies of the oracle's code with
one plausible error, on the CPU), which it must catch.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import as_f64


def _head(seed=5, T=9, S=6, D=8):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((T, S, D))
    k = rng.standard_normal((T, S, D)) / np.sqrt(D * S)
    v = rng.standard_normal((T, S, D))
    gamma = rng.uniform(0.9, 1.0, T)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    state = rng.standard_normal((D, D)) * 0.02
    return q, k, v, gamma, beta, state


FRAME_LISTS = [
    [0, 3, 8],          # sorted
    [7, 2, 5, 0],       # unsorted
    [4, 4, 1, 4, 8, 1], # repeated
    [8],                # the last frame alone
    [],                 # nothing
]


def _out_frames_pin(impl):
    """(ok, detail): impl(..., out_frames=F) equals rows F of the full output."""
    args = _head()
    full, MT = oracle.gdn_head(*args)
    for F in FRAME_LISTS:
        sub, sMT = impl(*args, out_frames=F)
        if sub.shape != (len(F),) + full.shape[1:]:
            return False, f"shape {sub.shape} for {F}"
        if not np.array_equal(sub, full[F]):
            return False, f"rows differ for out_frames={F}"
        if not np.array_equal(sMT, MT):
            return False, f"final state differs for out_frames={F}"
    return True, ""


def test_out_frames_equals_full_output_rows():
    ok, detail = _out_frames_pin(oracle.gdn_head)
    assert ok, detail


@pytest.mark.parametrize("bad", [[9], [-1], [0, 12]])
def test_out_frames_out_of_range_raises(bad):
    with pytest.raises(ValueError):
        oracle.gdn_head(*_head(), out_frames=bad)


# -- planted mistakes in copies of the subset path ----------------------------
def _subset_copy(select):
    """A copy of gdn_head's recurrence whose placement of the wanted outputs is
    `select(wanted, T) -> list of (frame, row)`."""
    def impl(q, k, v, gamma, beta, state=None, out_frames=None):
        q, k, v = as_f64(q), as_f64(k), as_f64(v)
        T, S, D = q.shape
        M = as_f64(state).copy()
        wanted = list(out_frames)
        O = np.zeros((len(wanted), S, D))
        place = select(wanted, T)
        for t in range(T):
            M = M @ (gamma[t] * (np.eye(D) - beta[t] * k[t].T @ k[t])) + beta[t] * v[t].T @ k[t]
            for f, i in place:
                if f == t:
                    O[i] = q[t] @ M.T
        return O, M
    return impl


SUBSET_MUTANTS = {
    # one slot per frame: a repeated frame fills only its last position
    "last_slot_wins": _subset_copy(lambda w, T: [(t, i) for t, i in {t: i for i, t in enumerate(w)}.items()]),
    # rows laid out in sorted frame order instead of the requested order
    "sorted_rows": _subset_copy(lambda w, T: [(t, i) for i, t in enumerate(sorted(w))]),
    # the output of the frame before the requested one
    "off_by_one": _subset_copy(lambda w, T: [(t - 1, i) for i, t in enumerate(w)]),
}


@pytest.mark.parametrize("name", sorted(SUBSET_MUTANTS))
def test_out_frames_pin_catches_mutant(name):
    ok, _ = _out_frames_pin(SUBSET_MUTANTS[name])
    assert not ok, f"mutant {name} passed the out_frames pin"


# -- the bf16 decode ----------------------------------------------------------
def _all_patterns():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _decode_pin(decode):
    """(ok, detail): decode(bits) equals torch's widening on every pattern
    (NaN patterns must decode to NaN)."""
    bits = _all_patterns()
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):
        got = np.asarray(decode(bits), dtype=np.float64)
    nan = np.isnan(ref)
    if not np.array_equal(np.isnan(got), nan):
        return False, "NaN patterns differ"
    bad = np.flatnonzero(got[~nan] != ref[~nan])
    if bad.size:
        return False, f"{bad.size} finite or infinite patterns differ"
    # signed zeros: -0.0 == 0.0 compares equal, so check the sign bit too
    if not np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])):
        return False, "signs differ"
    return True, ""


def test_as_f64_matches_torch_bf16_widening_on_every_pattern():
    ok, detail = _decode_pin(as_f64)
    assert ok, detail
    with np.errstate(invalid="ignore"):
        assert np.count_nonzero(~np.isnan(as_f64(_all_patterns()))) == 65536 - 254  # 2 * 127 NaN patterns


DECODE_MUTANTS = {
    "shift_15": lambda b: (b.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64),
    "as_float16": lambda b: b.view(np.float16).astype(np.float64),
    "as_integer": lambda b: b.astype(np.float64),
    "sign_dropped": lambda b: np.abs((b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)),
    "low_half": lambda b: b.astype(np.uint32).view(np.float32).astype(np.float64),
}


@pytest.mark.parametrize("name", sorted(DECODE_MUTANTS))
def test_decode_pin_catches_mutant(name):
    ok, _ = _decode_pin(DECODE_MUTANTS[name])
    assert not ok, f"mutant {name} passed the decode pin"
