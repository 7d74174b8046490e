"""Plain, slow fp64 CPU oracle for the backward pass (vector-Jacobian product)
of the frame-wise Gated DeltaNet forward.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or run anything in this directory.
The GPU library never calls it.

The pages describe training the model ("SANA-WM: NVIDIA puts a one-minute
world model on a single GPU", zhichai.net, training pipeline, Stages 1-4)
but give no backward formulas; the ones here are the exact derivative of the
forward that gdn_ref.py implements (same conventions: state rows are value
dims, columns key dims; one step per latent frame), derived by the chain
rule one operation at a time:

    G_t = K_t^T K_t,  U_t = V_t^T K_t,  A_t = gamma_t (I - beta_t G_t)
    M_t = M_{t-1} A_t + beta_t U_t,     O_t = Q_t M_t^T

Given the gradient dO_t of every output and dM_T of the final state, with
Lambda_t the total gradient reaching M_t:

    Lambda_t     = dO_t^T Q_t + (Lambda_{t+1} A_{t+1}^T)      (Lambda_{T+1} A^T := dM_T)
    dQ_t         = dO_t M_t
    dgamma_t     = < Lambda_t, M_{t-1} (I - beta_t G_t) >
    dbeta_t      = < Lambda_t, U_t - gamma_t M_{t-1} G_t >
    dG_t         = -gamma_t beta_t M_{t-1}^T Lambda_t
    dU_t         = beta_t Lambda_t
    dK_t         = V_t dU_t + K_t (dG_t + dG_t^T)
    dV_t         = K_t dU_t^T
    d(state_in)  = Lambda_1 A_1^T

(A_t is symmetric, so Lambda A^T = Lambda A.)  <X, Y> is the sum of the
elementwise products.  Everything is float64; bf16 inputs arrive as uint16 bit
patterns and are widened exactly.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .gdn_ref import as_f64, frame_maps, transition


def gdn_head_backward(q, k, v, gamma, beta, state=None, d_out=None,
                      d_state_out: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradients of one head.  q, k, v, d_out: [T, S, D]; gamma, beta: [T];
    state, d_state_out: [D, D] or None (zeros).  Returns dq, dk, dv [T, S, D],
    dgamma, dbeta [T] and dstate [D, D] (the gradient of state_in)."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    gamma, beta = as_f64(gamma), as_f64(beta)
    dO = as_f64(d_out)
    T, S, D = q.shape
    M0 = np.zeros((D, D)) if state is None else as_f64(state)

    # forward, keeping every state M_0 .. M_T and the per-frame maps
    Ms = [M0]
    Gs, Us = [], []
    for t in range(T):
        G, U = frame_maps(k[t], v[t])
        Gs.append(G)
        Us.append(U)
        Ms.append(Ms[-1] @ transition(G, gamma[t], beta[t]) + beta[t] * U)

    dq = np.empty((T, S, D))
    dk = np.empty((T, S, D))
    dv = np.empty((T, S, D))
    dgamma = np.empty(T)
    dbeta = np.empty(T)
    carry = np.zeros((D, D)) if d_state_out is None else as_f64(d_state_out).copy()
    for t in range(T - 1, -1, -1):
        M_prev, M_t, G, U = Ms[t], Ms[t + 1], Gs[t], Us[t]
        lam = carry + dO[t].T @ q[t]
        dq[t] = dO[t] @ M_t
        MG = M_prev @ G
        dgamma[t] = np.sum(lam * (M_prev - beta[t] * MG))
        dbeta[t] = np.sum(lam * (U - gamma[t] * MG))
        dG = -gamma[t] * beta[t] * (M_prev.T @ lam)
        dU = beta[t] * lam
        dk[t] = v[t] @ dU + k[t] @ (dG + dG.T)
        dv[t] = k[t] @ dU.T
        carry = lam @ transition(G, gamma[t], beta[t]).T
    return {"dq": dq, "dk": dk, "dv": dv, "dgamma": dgamma, "dbeta": dbeta, "dstate": carry}


def scalar_loss(q, k, v, gamma, beta, state, d_out, d_state_out=None) -> float:
    """<d_out, O> + <d_state_out, M_T>: the loss whose gradient
    gdn_head_backward returns (used by the finite-difference pin)."""
    from .gdn_ref import gdn_head
    O, M = gdn_head(q, k, v, gamma, beta, state)
    val = float(np.sum(as_f64(d_out) * O))
    if d_state_out is not None:
        val += float(np.sum(as_f64(d_state_out) * M))
    return val
