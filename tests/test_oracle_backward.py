"""Pins of the fp64 backward oracle (oracle/gdn_bwd.py) to facts outside it (CPU only):
torch autograd on a forward written here with torch ops, central finite
differences of the scalar loss, a closed form at T = 1, linearity in the
incoming gradients, and planted mistakes that these must catch."""
import numpy as np
import pytest
import torch

import oracle
from oracle.gdn_bwd import gdn_head_backward, scalar_loss

KEYS = ("dq", "dk", "dv", "dgamma", "dbeta", "dstate")


def _case(seed, T=4, S=5, D=3, state=True, d_state=True):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = {
        "q": rng.standard_normal((T, S, D)),
        "k": rng.standard_normal((T, S, D)) / np.sqrt(D * S),
        "v": rng.standard_normal((T, S, D)),
        "gamma": rng.uniform(0.8, 1.0, T),
        "beta": rng.uniform(0.1, 1.0, T),
        "state": rng.standard_normal((D, D)) if state else None,
    }
    g = {"d_out": rng.standard_normal((T, S, D)),
         "d_state_out": rng.standard_normal((D, D)) if d_state else None}
    return x, g


def _autograd(x, g):
    """The forward as the definition states it, in torch float64; torch
    differentiates it independently of the hand-derived adjoint."""
    t = {k: (None if v is None else torch.tensor(v, dtype=torch.float64, requires_grad=True))
         for k, v in x.items()}
    T, S, D = x["q"].shape
    M = t["state"] if t["state"] is not None else torch.zeros((D, D), dtype=torch.float64)
    outs = []
    for i in range(T):
        K, V, Q = t["k"][i], t["v"][i], t["q"][i]
        A = t["gamma"][i] * (torch.eye(D, dtype=torch.float64) - t["beta"][i] * (K.T @ K))
        M = M @ A + t["beta"][i] * (V.T @ K)
        outs.append(Q @ M.T)
    loss = (torch.stack(outs) * torch.tensor(g["d_out"])).sum()
    if g["d_state_out"] is not None:
        loss = loss + (M * torch.tensor(g["d_state_out"])).sum()
    loss.backward()
    names = {"dq": "q", "dk": "k", "dv": "v", "dgamma": "gamma", "dbeta": "beta", "dstate": "state"}
    return {k: (t[n].grad.numpy() if t[n] is not None else None) for k, n in names.items()}


@pytest.mark.parametrize("seed,state,d_state", [(1, True, True), (2, False, True), (3, True, False),
                                                (4, False, False)])
def test_backward_matches_torch_autograd(seed, state, d_state):
    x, g = _case(seed, state=state, d_state=d_state)
    ref = _autograd(x, g)
    got = gdn_head_backward(**x, **g)
    for key in KEYS:
        if ref[key] is None:
            continue
        assert np.allclose(got[key], ref[key], rtol=1e-11, atol=1e-12), key


def test_backward_matches_finite_differences():
    x, g = _case(7, T=3, S=4, D=3)
    got = gdn_head_backward(**x, **g)
    rng = np.random.Generator(np.random.PCG64(8))
    h = 1e-6
    names = {"q": "dq", "k": "dk", "v": "dv", "gamma": "dgamma", "beta": "dbeta", "state": "dstate"}
    for name, gkey in names.items():
        for _ in range(4):
            idx = tuple(int(rng.integers(0, n)) for n in x[name].shape)
            xp = {k: (None if v is None else v.copy()) for k, v in x.items()}
            xm = {k: (None if v is None else v.copy()) for k, v in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            fd = (scalar_loss(**xp, **g) - scalar_loss(**xm, **g)) / (2 * h)
            assert abs(fd - got[gkey][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, got[gkey][idx])


def test_single_frame_zero_state_closed_form():
    """T = 1, M_0 = 0: M_1 = beta U, O = beta Q U^T, so the loss is
    beta (<dO, Q U^T> + <dM, U>): dgamma = 0, dbeta = <dO, Q U^T> + <dM, U>,
    dQ = beta dO U, d(state_in) = gamma (Lambda - beta Lambda G) with
    Lambda = dO^T Q + dM."""
    x, g = _case(11, T=1, S=6, D=4, state=False)
    got = gdn_head_backward(**x, **g)
    K, V, Q = x["k"][0], x["v"][0], x["q"][0]
    dO, dM = g["d_out"][0], g["d_state_out"]
    U, G = V.T @ K, K.T @ K
    b, gm = x["beta"][0], x["gamma"][0]
    assert got["dgamma"][0] == 0.0
    assert np.isclose(got["dbeta"][0], np.sum(dO * (Q @ U.T)) + np.sum(dM * U), rtol=1e-13)
    assert np.allclose(got["dq"][0], b * dO @ U, rtol=1e-13)
    lam = dO.T @ Q + dM
    assert np.allclose(got["dstate"], gm * (lam - b * lam @ G), rtol=1e-13)


def test_backward_is_linear_in_incoming_gradients():
    x, g1 = _case(21)
    _, g2 = _case(22)
    a = gdn_head_backward(**x, **g1)
    b = gdn_head_backward(**x, **g2)
    c = gdn_head_backward(**x, d_out=g1["d_out"] + 2 * g2["d_out"],
                          d_state_out=g1["d_state_out"] + 2 * g2["d_state_out"])
    for key in KEYS:
        assert np.allclose(c[key], a[key] + 2 * b[key], rtol=1e-12, atol=1e-13), key


# ---- planted mistakes -------------------------------------------------------
def _mutant(kind):
    """The oracle's backward with one plausible mistake planted."""
    from oracle.gdn_ref import as_f64, frame_maps, transition

    def bwd(q, k, v, gamma, beta, state=None, d_out=None, d_state_out=None):
        q, k, v, gamma, beta, dO = map(as_f64, (q, k, v, gamma, beta, d_out))
        T, S, D = q.shape
        Ms = [np.zeros((D, D)) if state is None else as_f64(state)]
        Gs, Us = [], []
        for t in range(T):
            G, U = frame_maps(k[t], v[t])
            Gs.append(G)
            Us.append(U)
            Ms.append(Ms[-1] @ transition(G, gamma[t], beta[t]) + beta[t] * U)
        out = {n: np.empty((T, S, D)) for n in ("dq", "dk", "dv")}
        out["dgamma"], out["dbeta"] = np.empty(T), np.empty(T)
        carry = np.zeros((D, D)) if d_state_out is None else as_f64(d_state_out).copy()
        for t in range(T - 1, -1, -1):
            M_prev = Ms[t + 1] if kind == "state_after" else Ms[t]
            G, U = Gs[t], Us[t]
            lam = carry + dO[t].T @ q[t]
            out["dq"][t] = dO[t] @ (Ms[t + 1].T if kind == "dq_transposed" else Ms[t + 1])
            MG = M_prev @ G
            out["dgamma"][t] = np.sum(lam * (M_prev - beta[t] * MG))
            out["dbeta"][t] = np.sum(lam * (U - (1.0 if kind == "no_gamma_in_dbeta" else gamma[t]) * MG))
            dG = -gamma[t] * beta[t] * (M_prev.T @ lam)
            dU = beta[t] * lam
            sym = dG if kind == "no_symmetrize" else dG + dG.T
            out["dk"][t] = v[t] @ dU + k[t] @ sym
            out["dv"][t] = k[t] @ (dU if kind == "dv_untransposed" else dU.T)
            A = transition(G, gamma[t], beta[t])
            carry = lam @ (np.eye(D) if kind == "no_carry_transition" else A.T)
        out["dstate"] = carry
        return out
    return bwd


@pytest.mark.parametrize("kind", ["state_after", "dq_transposed", "no_gamma_in_dbeta", "no_symmetrize",
                                  "dv_untransposed", "no_carry_transition"])
def test_pins_catch_planted_mistakes(kind):
    x, g = _case(31, T=3, S=4, D=3)
    ref = _autograd(x, g)
    got = _mutant(kind)(**x, **g)
    assert any(not np.allclose(got[k], ref[k], rtol=1e-9, atol=1e-10) for k in KEYS)


def test_unmutated_copy_passes():
    x, g = _case(31, T=3, S=4, D=3)
    ref = _autograd(x, g)
    got = _mutant("none")(**x, **g)
    assert all(np.allclose(got[k], ref[k], rtol=1e-11, atol=1e-12) for k in KEYS)
