"""The form of one step that the single-frame kernel computes, checked in
float64 against the oracle (which follows the pages' G/U form).

One step M' = gamma (M - beta M G) + beta U with G = K^T K and U = V^T K
(zhichai.net, section 1) equals, with G and U written out over the frame's
tokens s,
    M' = gamma M + beta sum_s (v_s - gamma M k_s) k_s^T,
and with the keys scaled by ks, M' = gamma M + beta ks sum_s
(v_s - gamma ks M k_s) k_s^T (the delta rule written literally, as in
oracle.gdn_head_residual).  Rows of M' then depend only on the same rows
of M and the same columns of V, and O[:, r] = Q M'_r^T needs only rows r
of M': the kernel gives each 16-row block to one workgroup.  These tests
write the step out per token, with the key scale where the kernel applies
it, compare it with oracle.gdn_head on a single frame, and check the
row-block independence on its own (with everything outside the block
replaced by NaN)."""
import numpy as np
import pytest

import oracle


def _frame(seed, S=37, D=32, state=True):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((1, S, D))
    k = rng.standard_normal((1, S, D)) / np.sqrt(D * S)
    v = rng.standard_normal((1, S, D))
    gamma = rng.uniform(0.9, 1.0, 1)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(1)))
    M = rng.standard_normal((D, D)) * 0.05 if state else None
    return q, k, v, gamma, beta, M


def _per_token_step(q, k, v, gamma, beta, M, ks=1.0):
    """The single-frame kernel's arithmetic in float64: residual of every
    token against the decayed state, times its key."""
    D = k.shape[-1]
    M = np.zeros((D, D)) if M is None else M
    g, b = float(gamma[0]), float(beta[0])
    P = np.zeros((D, D))
    for s in range(k.shape[1]):
        ks_vec = k[0, s]
        r = v[0, s] - g * ks * (M @ ks_vec)
        P += np.outer(r, ks_vec)
    M_new = g * M + b * ks * P
    return q[0] @ M_new.T, M_new


@pytest.mark.parametrize("seed,state", [(1, True), (2, False), (3, True)])
def test_per_token_form_equals_oracle_step(seed, state):
    q, k, v, gamma, beta, M = _frame(seed, state=state)
    O_ref, M_ref = oracle.gdn_head(q, k, v, gamma, beta, M)
    O, M_new = _per_token_step(q, k, v, gamma, beta, M)
    assert np.allclose(M_new, M_ref, rtol=0, atol=1e-12 * np.abs(M_ref).max())
    assert np.allclose(O, O_ref[0], rtol=0, atol=1e-12 * np.abs(O_ref).max())


def test_per_token_form_with_key_scale():
    """Raw keys with the scale applied in the step equal the oracle on scaled keys."""
    q, k, v, gamma, beta, M = _frame(4)
    ks = 0.37
    O_ref, M_ref = oracle.gdn_head(q, ks * k, v, gamma, beta, M)
    O, M_new = _per_token_step(q, k, v, gamma, beta, M, ks=ks)
    assert np.allclose(M_new, M_ref, rtol=0, atol=1e-12 * np.abs(M_ref).max())
    assert np.allclose(O, O_ref[0], rtol=0, atol=1e-12 * np.abs(O_ref).max())


def test_row_blocks_are_independent():
    """Rows r of M' from rows r of M and columns r of V alone; output
    columns r from rows r of M' alone."""
    q, k, v, gamma, beta, M = _frame(5, D=32)
    O, M_new = _per_token_step(q, k, v, gamma, beta, M)
    rows = slice(16, 32)
    # everything outside the block replaced by garbage
    M_bad = np.full_like(M, np.nan)
    M_bad[rows] = M[rows]
    v_bad = np.full_like(v, np.nan)
    v_bad[..., rows] = v[..., rows]
    g, b = float(gamma[0]), float(beta[0])
    P_r = sum(np.outer(v_bad[0, s, rows] - g * (M_bad[rows] @ k[0, s]), k[0, s]) for s in range(k.shape[1]))
    M_r = g * M_bad[rows] + b * P_r
    assert np.allclose(M_r, M_new[rows], rtol=0, atol=1e-12)
    assert np.allclose(q[0] @ M_r.T, O[:, rows], rtol=0, atol=1e-12)


def test_form_catches_a_dropped_decay():
    """A plausible slip (the decay left out of the prediction) is caught."""
    q, k, v, gamma, beta, M = _frame(6)
    _, M_ref = oracle.gdn_head(q, k, v, gamma, beta, M)
    g, b = float(gamma[0]), float(beta[0])
    P = sum(np.outer(v[0, s] - (M @ k[0, s]), k[0, s]) for s in range(k.shape[1]))
    M_slip = g * M + b * P
    assert not np.allclose(M_slip, M_ref, rtol=0, atol=1e-12 * np.abs(M_ref).max())
