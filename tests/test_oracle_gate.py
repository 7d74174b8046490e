"""Pins for the gate prologue's oracle (oracle/gate_ref.py): gamma_t and
beta_t of each frame from per-token pre-activations.  Each pin ties it to
something outside it:
* closed forms: zero pre-activations and parameters give gamma = beta = 1/2;
  softplus(ln(e - 1)) = 1 gives gamma = exp(-exp(A_log)); large negative
  inputs give gamma -> 1;
* library routines: torch's softplus and sigmoid in float64 on random inputs;
* structure: a frame's gates depend on its tokens only through their mean
  (token order and a constant shift folded into dt_bias), gamma decreases
  and beta increases with their pre-activations, both stay in (0, 1).
Planted mistakes must each be caught.
"""
import numpy as np
import pytest
import torch

from oracle.gate_ref import frame_gates, gdn_head_gated
from oracle import gdn_head


def _rand(T=6, S=11, seed=0, scale=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((T, S)) * scale, rng.standard_normal((T, S)) * scale


def pin_zero(fg):
    g, b = fg(np.zeros((3, 5)), np.zeros((3, 5)), 0.0, 0.0)
    return np.allclose(g, 0.5, rtol=0, atol=1e-15) and np.allclose(b, 0.5, rtol=0, atol=1e-15), "zero inputs"


def pin_unit_softplus(fg):
    bias = np.log(np.e - 1.0)  # softplus(bias) = 1
    for A_log in (-1.0, 0.0, 0.7):
        g, _ = fg(np.zeros((2, 4)), np.zeros((2, 4)), A_log, bias)
        if not np.allclose(g, np.exp(-np.exp(A_log)), rtol=1e-14, atol=0):
            return False, f"A_log {A_log}"
    g, _ = fg(np.full((1, 3), -60.0), np.zeros((1, 3)), 0.0, 0.0)
    return bool(abs(g[0] - 1.0) < 1e-20 + 1e-25 and g[0] <= 1.0), "large negative pre-activation"


def pin_torch(fg):
    a, b = _rand(seed=1, scale=3.0)
    A_log, bias = 0.3, -0.4
    g, bt = fg(a, b, A_log, bias)
    ta, tb = torch.from_numpy(a).mean(dim=1), torch.from_numpy(b).mean(dim=1)
    tg = torch.exp(-np.exp(A_log) * torch.nn.functional.softplus(ta + bias))
    ok = np.allclose(g, tg.numpy(), rtol=1e-14, atol=0) and np.allclose(bt, torch.sigmoid(tb).numpy(), rtol=1e-14,
                                                                       atol=0)
    return ok, "torch softplus / sigmoid"


def pin_mean_pooling(fg):
    a, b = _rand(seed=2)
    g, bt = fg(a, b, 0.1, 0.2)
    perm = np.random.Generator(np.random.PCG64(3)).permutation(a.shape[1])
    g2, b2 = fg(a[:, perm], b[:, perm], 0.1, 0.2)
    g3, _ = fg(a + 0.5, b, 0.1, 0.2 - 0.5)  # a constant shift of every token = a shift of dt_bias
    ok = (np.allclose(g, g2, rtol=1e-14, atol=0) and np.allclose(bt, b2, rtol=1e-14, atol=0)
          and np.allclose(g, g3, rtol=1e-13, atol=0))
    return ok, "mean pooling"


def pin_monotone(fg):
    xs = np.linspace(-6, 6, 25)[:, None] * np.ones((1, 3))
    g, b = fg(xs, xs, 0.2, 0.1)
    ok = (np.all(np.diff(g) < 0) and np.all(np.diff(b) > 0) and np.all((g > 0) & (g < 1))
          and np.all((b > 0) & (b < 1)))
    gA, _ = fg(np.zeros((1, 2)), np.zeros((1, 2)), 1.0, 0.0)
    gB, _ = fg(np.zeros((1, 2)), np.zeros((1, 2)), 0.0, 0.0)
    return bool(ok and gA[0] < gB[0]), "monotone and bounded"


PINS = {"zero": pin_zero, "unit_softplus": pin_unit_softplus, "torch": pin_torch, "mean": pin_mean_pooling,
        "monotone": pin_monotone}


@pytest.mark.parametrize("name", sorted(PINS))
def test_gate_pin(name):
    ok, detail = PINS[name](frame_gates)
    assert ok, detail


def test_gated_forward_is_the_forward_on_its_gates_and_scaled_keys():
    rng = np.random.Generator(np.random.PCG64(4))
    T, S, D = 5, 7, 6
    q, k, v = (rng.standard_normal((T, S, D)) for _ in range(3))
    a, b = _rand(T, S, seed=5)
    ks = 1 / np.sqrt(D * S)
    O, M, g, bt = gdn_head_gated(q, k, v, a, b, -0.2, 0.3, key_scale=ks)
    O2, M2 = gdn_head(q, k * ks, v, *frame_gates(a, b, -0.2, 0.3))
    assert np.array_equal(O, O2) and np.array_equal(M, M2)


def _mut(kind):
    def fg(gate_a, gate_b, A_log, dt_bias):
        a, b = np.asarray(gate_a, float), np.asarray(gate_b, float)
        am, bm = a.mean(axis=1), b.mean(axis=1)
        sp = np.logaddexp(0.0, am + dt_bias)
        if kind == "sum_not_mean":
            am, bm = a.sum(axis=1), b.sum(axis=1)
            sp = np.logaddexp(0.0, am + dt_bias)
        elif kind == "relu_not_softplus":
            sp = np.maximum(am + dt_bias, 0.0)
        elif kind == "bias_after_softplus":
            sp = np.logaddexp(0.0, am) + dt_bias
        g = np.exp(-np.exp(A_log) * sp)
        if kind == "sign":
            g = np.exp(np.exp(A_log) * sp)
        elif kind == "A_log_not_exponentiated":
            g = np.exp(-A_log * sp)
        bt = 1 / (1 + np.exp(-bm))
        if kind == "one_minus_beta":
            bt = 1 - bt
        elif kind == "beta_from_a":
            bt = 1 / (1 + np.exp(-am))
        elif kind == "max_pool":
            g = np.exp(-np.exp(A_log) * np.logaddexp(0.0, a.max(axis=1) + dt_bias))
        return g, bt
    return fg


MUTANTS = ["sum_not_mean", "relu_not_softplus", "bias_after_softplus", "sign", "A_log_not_exponentiated",
           "one_minus_beta", "beta_from_a", "max_pool"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_gate_pins_catch_mutant(kind):
    with np.errstate(all="ignore"):
        res = {n: bool(p(_mut(kind))[0]) for n, p in PINS.items()}
    assert not all(res.values()), f"mutant {kind} passed every pin"
