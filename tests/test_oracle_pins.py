"""Pins of the fp64 oracle to facts fixed outside it (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact
from synth import TINY_F32, CLIP_5S, STRESS_B4, head_inputs

from pins import all_checks, load_case, exact_cases, check_golden

IMPLS = {"recurrence": oracle.gdn_head, "residual_form": oracle.gdn_head_residual}


@pytest.mark.parametrize("impl_name", sorted(IMPLS))
def test_all_pins_pass(impl_name):
    res = all_checks(IMPLS[impl_name], oracle.tokenwise_gated_delta)
    bad = {k: v for k, v in res.items() if not v[0]}
    assert not bad, bad


@pytest.mark.parametrize("name", ["hand_d1.json", "hand_d2.json"])
def test_exact_bruteforce_matches_hand_examples(name):
    """The exact closed form reproduces the hand-worked fixtures exactly."""
    import json, os
    from pins import GOLDEN
    with open(os.path.join(GOLDEN, name)) as f:
        c = json.load(f)
    O, M = exact.unrolled(c["q"], c["k"], c["v"], c["gamma"], c["beta"], c["state"])
    assert [[str(x) for x in r] for r in M] == [[str(Fraction(x)) for x in r] for r in c["M_T"]]
    for t in range(c["T"]):
        assert [[Fraction(x) for x in r] for r in O[t]] == [[Fraction(x) for x in r] for r in c["O"][t]]


def test_exact_golden_file_is_reproducible():
    """The stored exact fixture still equals what the exact brute force gives."""
    for c in exact_cases():
        O, M = exact.unrolled(c["q"], c["k"], c["v"], c["gamma"], c["beta"], c["state"])
        assert [[str(x) for x in r] for r in M] == c["M_T"]
        assert [[[str(x) for x in r] for r in Ot] for Ot in O] == c["O"]


def test_bruteforce_random_dyadic_bitwise():
    """Fresh random dyadic cases: fp64 recurrence == exact closed form, bit for bit."""
    rng = np.random.Generator(np.random.PCG64(99))
    for T, S, D in [(3, 2, 2), (4, 3, 3), (2, 4, 2), (4, 1, 3)]:
        dy = lambda *shape: rng.integers(-8, 9, size=shape) / 4.0
        q, k, v = dy(T, S, D), dy(T, S, D), dy(T, S, D)
        gamma = rng.integers(2, 5, size=T) / 4.0
        beta = rng.integers(0, 5, size=T) / 4.0
        M0 = dy(D, D)
        O, M = oracle.gdn_head(q, k, v, gamma, beta, M0)
        Oe, Me = exact.unrolled(q.tolist(), k.tolist(), v.tolist(), gamma.tolist(), beta.tolist(), M0.tolist())
        Me = np.array([[float(x) for x in r] for r in Me])
        Oe = np.array([[[float(x) for x in r] for r in Ot] for Ot in Oe])
        assert np.array_equal(M, Me) and np.array_equal(O, Oe)


@pytest.mark.parametrize("chunk", [1, 2, 3, 5, 8, 64])
def test_prefix_composition_equals_sequential(chunk):
    """Composing the per-frame affine maps over chunks gives the same states
    (zhichai.net page, Stage 3: prefix-sum composition is exact)."""
    rng = np.random.Generator(np.random.PCG64(7))
    T, S, D = 13, 6, 5
    k = rng.standard_normal((T, S, D)) / np.sqrt(D * S)
    v = rng.standard_normal((T, S, D))
    gamma = rng.uniform(0.9, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    M0 = rng.standard_normal((D, D))
    G, U = oracle.build_maps_head(k, v)
    seq = oracle.state_pass_head(G, U, gamma, beta, M0)
    chk = oracle.state_pass_chunked(G, U, gamma, beta, M0, chunk=chunk)
    np.testing.assert_allclose(chk, seq, rtol=1e-13, atol=1e-14)


def test_stage_functions_compose_to_forward():
    rng = np.random.Generator(np.random.PCG64(8))
    T, S, D = 6, 9, 4
    q, k, v = (rng.standard_normal((T, S, D)) for _ in range(3))
    gamma = rng.uniform(0.9, 1.0, T)
    beta = rng.uniform(0, 1, T)
    M0 = rng.standard_normal((D, D))
    O, M, states = oracle.gdn_head(q, k, v, gamma, beta, M0, keep_states=True)
    G, U = oracle.build_maps_head(k, v)
    st = oracle.state_pass_head(G, U, gamma, beta, M0)
    np.testing.assert_allclose(st, states, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(oracle.output_head(q, st), O, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(states[-1], M)


def test_residual_form_agrees_on_tiny_workload():
    w = TINY_F32
    d = head_inputs(w, 0, 1)
    O1, M1 = oracle.gdn_head(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["state"])
    O2, M2 = oracle.gdn_head_residual(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["state"])
    np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(M2, M1, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("w", [CLIP_5S.with_(T=3), STRESS_B4.with_(T=3)], ids=["clip5s", "stress"])
def test_key_scaling_bounds_transition_on_workloads(w):
    """With keys pre-scaled by 1/sqrt(D*S), every generated frame has
    lambda_max(K^T K) <= 2/beta, so ||I - beta K^T K||_2 <= 1 (zhichai.net page,
    section 1: the scaling bounds the transition's spectral norm)."""
    d = head_inputs(w, 0, 0)
    k = oracle.as_f64(d["k"])
    for t in range(w.T):
        G = k[t].T @ k[t]
        lam = np.linalg.eigvalsh(G)
        assert lam.min() >= -1e-12
        assert lam.max() <= 2.0 / d["beta"][t]
        A = np.eye(w.D) - d["beta"][t] * G
        assert np.linalg.norm(A, 2) <= 1.0 + 1e-12


def test_oracle_counts():
    assert oracle.flops_per_head_frame(880, 128) == 90_701_824


def test_no_frames_leaves_the_state():
    """T = 0: no step is taken, so M_T = M_0 and O has no frames."""
    rng = np.random.Generator(np.random.PCG64(31))
    D, S = 4, 3
    M0 = rng.standard_normal((D, D))
    empty = np.zeros((0, S, D))
    O, M = oracle.gdn_head(empty, empty, empty, np.zeros(0), np.zeros(0), M0)
    assert O.shape == (0, S, D) and np.array_equal(M, M0)
    O, M = oracle.gdn_head(empty, empty, empty, np.zeros(0), np.zeros(0), None)
    assert np.array_equal(M, np.zeros((D, D)))


def test_frames_without_tokens_only_decay():
    """S = 0: K_t has no rows, so G_t = U_t = 0 and M_t = gamma_t M_{t-1}
    whatever beta is; the state after T frames is prod(gamma) M_0."""
    rng = np.random.Generator(np.random.PCG64(32))
    T, D = 6, 5
    M0 = rng.standard_normal((D, D))
    gamma = rng.uniform(0.5, 1.0, T)
    beta = rng.uniform(-1.0, 2.0, T)
    empty = np.zeros((T, 0, D))
    O, M = oracle.gdn_head(empty, empty, empty, gamma, beta, M0)
    assert O.shape == (T, 0, D)
    assert np.allclose(M, np.prod(gamma) * M0, rtol=1e-14, atol=0)


def test_backward_of_frames_without_tokens_closed_form():
    """S = 0, loss <dM_T, M_T> with M_T = prod(gamma) M_0:
    dgamma_t = prod_{u != t} gamma_u <dM_T, M_0>, dbeta = 0,
    d(state_in) = prod(gamma) dM_T."""
    rng = np.random.Generator(np.random.PCG64(33))
    T, D = 5, 4
    M0, dM = rng.standard_normal((D, D)), rng.standard_normal((D, D))
    gamma = rng.uniform(0.5, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    empty = np.zeros((T, 0, D))
    g = oracle.gdn_head_backward(empty, empty, empty, gamma, beta, M0, empty, dM)
    dot = float(np.sum(dM * M0))
    want = np.array([np.prod(np.delete(gamma, t)) * dot for t in range(T)])
    assert np.allclose(g["dgamma"], want, rtol=1e-13, atol=0)
    assert np.array_equal(g["dbeta"], np.zeros(T))
    assert np.allclose(g["dstate"], np.prod(gamma) * dM, rtol=1e-14, atol=0)
    for key in ("dq", "dk", "dv"):
        assert g[key].shape == (T, 0, D)
    # no frames: the incoming state gradient passes through unchanged
    none = np.zeros((0, 0, D))
    g0 = oracle.gdn_head_backward(none, none, none, np.zeros(0), np.zeros(0), M0, none, dM)
    assert np.array_equal(g0["dstate"], dM)
