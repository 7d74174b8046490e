"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch each one.  This is what shows the pins are not vacuous."""
import numpy as np
import pytest

import oracle
from oracle import as_f64
from pins import all_checks


def _make(step, out_before=False):
    """A gdn_head variant whose per-frame update is `step(M, K, V, gamma, beta)`."""
    def impl(q, k, v, gamma, beta, state=None):
        q, k, v = as_f64(q), as_f64(k), as_f64(v)
        T, S, D = q.shape
        M = np.zeros((D, D)) if state is None else as_f64(state).copy()
        O = np.empty((T, S, D))
        for t in range(T):
            Mprev = M
            M = step(M, k[t], v[t], gamma[t], beta[t])
            O[t] = q[t] @ (Mprev if out_before else M).T
        return O, M
    return impl


I = lambda d: np.eye(d)

MUTANTS = {
    # decay dropped from the transition
    "no_gamma": _make(lambda M, K, V, g, b: M @ (I(len(M)) - b * K.T @ K) + b * V.T @ K),
    # gamma also scales the injection
    "gamma_on_injection": _make(lambda M, K, V, g, b: g * (M @ (I(len(M)) - b * K.T @ K) + b * V.T @ K)),
    # wrong sign of the delta-rule term
    "plus_beta": _make(lambda M, K, V, g, b: M @ (g * (I(len(M)) + b * K.T @ K)) + b * V.T @ K),
    # transition applied on the wrong side
    "A_times_M": _make(lambda M, K, V, g, b: (g * (I(len(M)) - b * K.T @ K)) @ M + b * V.T @ K),
    # injection transposed
    "KtV": _make(lambda M, K, V, g, b: M @ (g * (I(len(M)) - b * K.T @ K)) + b * K.T @ V),
    # beta dropped from the injection
    "no_beta_injection": _make(lambda M, K, V, g, b: M @ (g * (I(len(M)) - b * K.T @ K)) + V.T @ K),
    # beta dropped from the transition
    "no_beta_transition": _make(lambda M, K, V, g, b: M @ (g * (I(len(M)) - K.T @ K)) + b * V.T @ K),
    # Gram matrix taken over the wrong axis (token x token is not D x D; use K K^T trimmed) -> use V^T V
    "gram_of_values": _make(lambda M, K, V, g, b: M @ (g * (I(len(M)) - b * V.T @ V)) + b * V.T @ K),
    # output read from the state before the frame's update
    "output_before_update": _make(lambda M, K, V, g, b: M @ (g * (I(len(M)) - b * K.T @ K)) + b * V.T @ K,
                                  out_before=True),
}


def _transposed_output(q, k, v, gamma, beta, state=None):
    O, M = oracle.gdn_head(q, k, v, gamma, beta, state)
    # O_t = Q_t M_t instead of Q_t M_t^T
    q64 = as_f64(q)
    _, _, states = oracle.gdn_head(q, k, v, gamma, beta, state, keep_states=True)
    return np.einsum("tsj,tji->tsi", q64, states), M


def _state_as_transpose(q, k, v, gamma, beta, state=None):
    O, M = oracle.gdn_head(q, k, v, gamma, beta, state)
    return O, M.T


MUTANTS["output_without_transpose"] = _transposed_output
MUTANTS["state_returned_transposed"] = _state_as_transpose


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    res = all_checks(MUTANTS[name], oracle.tokenwise_gated_delta, exact=False)
    failed = [k for k, (ok, _) in res.items() if not ok]
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes():
    ref = _make(lambda M, K, V, g, b: M @ (g * (I(len(M)) - b * K.T @ K)) + b * V.T @ K)
    res = all_checks(ref, oracle.tokenwise_gated_delta, exact=True)
    assert all(ok for ok, _ in res.values()), {k: v for k, v in res.items() if not v[0]}
