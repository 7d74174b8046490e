"""Checks that pin a frame-wise GDN implementation to facts fixed outside it.

Each check takes `impl`, a callable with the signature of
oracle.gdn_head(q, k, v, gamma, beta, state) -> (O [T,S,D], M_T [D,D]) working
on float64 arrays, and returns (ok: bool, detail: str).  The pin tests run
them on the oracle and require every one to pass; the mutation tests run them
on deliberately broken copies of the oracle and require at least one to fail.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac_array(x):
    return np.array(x, dtype=object)


def _to_f64(x):
    if x is None:
        return None
    return np.vectorize(lambda e: float(Fraction(e)), otypes=[np.float64])(np.array(x, dtype=object))


def load_case(path_or_case):
    c = path_or_case
    if isinstance(c, str):
        with open(os.path.join(GOLDEN, c)) as f:
            c = json.load(f)
    out = {key: _to_f64(c[key]) for key in ("q", "k", "v", "gamma", "beta", "O", "M_T")}
    out["state"] = _to_f64(c["state"])
    return out


def exact_cases():
    with open(os.path.join(GOLDEN, "exact_unrolled.json")) as f:
        return json.load(f)["cases"]


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _rand_head(rng, T, S, D, scale_keys=True, state=True):
    q = rng.standard_normal((T, S, D))
    k = rng.standard_normal((T, S, D))
    if scale_keys:
        k /= np.sqrt(D * S)
    v = rng.standard_normal((T, S, D))
    gamma = rng.uniform(0.8, 1.0, T)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    M0 = rng.standard_normal((D, D)) * 0.3 if state else None
    return q, k, v, gamma, beta, M0


# ---------------------------------------------------------------------------
def check_golden(impl, name):
    """Hand-worked or exact-rational fixtures: dyadic inputs keep every fp64
    operation exact, so the result must equal the stored fractions exactly."""
    c = load_case(name) if isinstance(name, str) else load_case(name)
    O, M = impl(c["q"], c["k"], c["v"], c["gamma"], c["beta"], c["state"])
    ok = np.array_equal(O, c["O"]) and np.array_equal(M, c["M_T"])
    return ok, f"max|dO|={np.max(np.abs(O - c['O'])):.3g} max|dM|={np.max(np.abs(M - c['M_T'])):.3g}"


def check_identity(impl, seed=11):
    """gamma=1, beta=0: the state never changes and O_t = Q_t M_0^T."""
    q, k, v, _, _, M0 = _rand_head(_rng(seed), 5, 7, 4)
    T = q.shape[0]
    O, M = impl(q, k, v, np.ones(T), np.zeros(T), M0)
    ok = np.allclose(M, M0, rtol=0, atol=1e-14) and np.allclose(O, q @ M0.T, rtol=0, atol=1e-13)
    return ok, "identity"


def check_pure_decay(impl, seed=12):
    """beta=0: M_t = (prod_{u<=t} gamma_u) M_0 (pure geometric decay)."""
    q, k, v, gamma, _, M0 = _rand_head(_rng(seed), 6, 5, 3)
    T = q.shape[0]
    O, M = impl(q, k, v, gamma, np.zeros(T), M0)
    scale = np.cumprod(gamma)
    ok = np.allclose(M, scale[-1] * M0, rtol=1e-13, atol=1e-15)
    for t in range(T):
        ok &= np.allclose(O[t], scale[t] * (q[t] @ M0.T), rtol=1e-12, atol=1e-14)
    return bool(ok), "pure decay"


def check_no_residual(impl, seed=13):
    """gamma=1 and V_t = K_t M_{t-1}^T (the target equals the prediction):
    the delta rule has nothing to correct, so M stays M_0 for any beta."""
    rng = _rng(seed)
    q, k, _, _, beta, M0 = _rand_head(rng, 5, 6, 4)
    T = q.shape[0]
    v = np.einsum("tsj,ij->tsi", k, M0)
    beta = rng.uniform(0.1, 1.0, T)
    O, M = impl(q, k, v, np.ones(T), beta, M0)
    ok = np.allclose(M, M0, rtol=0, atol=1e-13)
    return ok, f"max|M-M0|={np.max(np.abs(M - M0)):.3g}"


def check_overwrite(impl, seed=14):
    """gamma=beta=1 and orthonormal key columns (K_t^T K_t = I): the transition
    vanishes, M_t = V_t^T K_t, and with square K_t = Q_t the frame is read back
    exactly, O_t = V_t."""
    rng = _rng(seed)
    T, D = 3, 4
    S = D
    k = np.stack([np.linalg.qr(rng.standard_normal((S, D)))[0] for _ in range(T)])
    v = rng.standard_normal((T, S, D))
    M0 = rng.standard_normal((D, D))
    O, M = impl(k.copy(), k, v, np.ones(T), np.ones(T), M0)
    ok = np.allclose(M, v[-1].T @ k[-1], atol=1e-12) and np.allclose(O, v, atol=1e-12)
    return ok, f"max|O-V|={np.max(np.abs(O - v)):.3g}"


def check_tokenwise(impl, tokenwise, seed=15):
    """S=1: each frame is one token, so the frame-wise rule is the textbook
    token-wise gated delta rule with outer products k k^T and v k^T."""
    q, k, v, gamma, beta, M0 = _rand_head(_rng(seed), 9, 1, 5)
    O, M = impl(q, k, v, gamma, beta, M0)
    o2, M2 = tokenwise(q[:, 0], k[:, 0], v[:, 0], gamma, beta, M0)
    ok = np.allclose(O[:, 0], o2, rtol=1e-12, atol=1e-13) and np.allclose(M, M2, rtol=1e-12, atol=1e-13)
    return ok, "token-wise"


def check_streaming(impl, seed=16):
    """Successive calls over frame ranges, carrying the state, equal one call."""
    q, k, v, gamma, beta, M0 = _rand_head(_rng(seed), 11, 6, 4)
    O, M = impl(q, k, v, gamma, beta, M0)
    parts, st, t0 = [], M0, 0
    for c in (4, 1, 5, 1):
        sl = slice(t0, t0 + c)
        o, st = impl(q[sl], k[sl], v[sl], gamma[sl], beta[sl], st)
        parts.append(o)
        t0 += c
    ok = np.allclose(np.concatenate(parts), O, rtol=1e-13, atol=1e-14) and np.allclose(st, M, rtol=1e-13, atol=1e-14)
    return ok, "streaming"


def check_linearity(impl, seed=17):
    """O is linear in Q; (O, M_T) are jointly linear in (V, M_0)."""
    rng = _rng(seed)
    q, k, v, gamma, beta, M0 = _rand_head(rng, 4, 5, 3)
    q2, _, v2, _, _, M02 = _rand_head(rng, 4, 5, 3)
    a, b = 0.7, -1.3
    O1, M1 = impl(q, k, v, gamma, beta, M0)
    O2, _ = impl(q2, k, v, gamma, beta, M0)
    O12, _ = impl(a * q + b * q2, k, v, gamma, beta, M0)
    ok = np.allclose(O12, a * O1 + b * O2, rtol=1e-12, atol=1e-12)
    Ov, Mv = impl(q, k, v2, gamma, beta, M02)
    Os, Ms = impl(q, k, v + v2, gamma, beta, M0 + M02)
    ok &= np.allclose(Os, O1 + Ov, rtol=1e-12, atol=1e-12) and np.allclose(Ms, M1 + Mv, rtol=1e-12, atol=1e-12)
    return bool(ok), "linearity"


def check_orientation(impl, seed=18):
    """T=1, M_0=0: M_1[i, j] = beta * sum_s V[s, i] K[s, j] (rows value, cols key),
    and O_1[s, i] = sum_j Q[s, j] M_1[i, j]; written as explicit loops."""
    rng = _rng(seed)
    S, D = 3, 4
    q, k, v = (rng.standard_normal((1, S, D)) for _ in range(3))
    beta = 0.625
    O, M = impl(q, k, v, np.array([0.9]), np.array([beta]), None)
    Mx = np.zeros((D, D))
    for i in range(D):
        for j in range(D):
            Mx[i, j] = beta * sum(v[0, s, i] * k[0, s, j] for s in range(S))
    Ox = np.zeros((S, D))
    for s in range(S):
        for i in range(D):
            Ox[s, i] = sum(q[0, s, j] * Mx[i, j] for j in range(D))
    ok = np.allclose(M, Mx, rtol=1e-13, atol=1e-15) and np.allclose(O[0], Ox, rtol=1e-13, atol=1e-15)
    return ok, "orientation"


def check_bounded(impl, seed=19):
    """With keys scaled by 1/sqrt(D*S), lambda_max(K^T K) <= 2/beta, hence
    ||A_t||_2 <= gamma_t <= 1 and ||M_t||_2 <= ||M_0||_2 + sum_u beta_u ||U_u||_2."""
    q, k, v, gamma, beta, M0 = _rand_head(_rng(seed), 8, 16, 8)
    O, M = impl(q, k, v, gamma, beta, M0)
    bound = np.linalg.norm(M0, 2) + sum(
        beta[t] * np.linalg.norm(v[t].T @ k[t], 2) for t in range(len(gamma)))
    ok = np.linalg.norm(M, 2) <= bound * (1 + 1e-12)
    return bool(ok), f"||M||={np.linalg.norm(M, 2):.4g} bound={bound:.4g}"


def all_checks(impl, tokenwise, exact=True):
    """Run every pin on `impl`; returns {name: (ok, detail)}."""
    res = {
        "golden_d1": check_golden(impl, "hand_d1.json"),
        "golden_d2": check_golden(impl, "hand_d2.json"),
        "identity": check_identity(impl),
        "pure_decay": check_pure_decay(impl),
        "no_residual": check_no_residual(impl),
        "overwrite": check_overwrite(impl),
        "tokenwise": check_tokenwise(impl, tokenwise),
        "streaming": check_streaming(impl),
        "linearity": check_linearity(impl),
        "orientation": check_orientation(impl),
        "bounded": check_bounded(impl),
    }
    if exact:
        for i, c in enumerate(exact_cases()):
            res[f"exact_{i}"] = check_golden(impl, c)
    return res
