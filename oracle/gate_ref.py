"""Plain fp64 CPU oracle for the gate prologue of the frame-wise GDN: the
decay gate gamma_t and the delta-rule strength beta_t of each frame computed
from activations, then the recurrence of gdn_ref.gdn_head.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or run anything in this directory.
The GPU library never calls it, and it imports nothing from the GPU package.

What the pages say ("SANA-WM: NVIDIA puts a one-minute world model on a
single GPU", zhichai.net): section 1 calls gamma a learned decay scalar that
multiplies the previous state and beta the strength of the delta-rule
correction; the training pipeline fuses "the GDN scan and gate operations"
into custom kernels.  They do not say how gamma and beta come from the
activations.  The reading taken here, the parameterisation of gated linear
recurrences with a learned log-rate per head, made frame-wise because one
recurrent step consumes a whole latent frame (bilibili cv49203711, fourth key
point):
  * the layer's projections give each token s of frame t two gate
    pre-activations a[t, s] and b[t, s] per head (inputs here);
  * a frame's gate inputs are their means over its S tokens;
  * gamma_t = exp(-exp(A_log) * softplus(mean_s a[t, s] + dt_bias)),
    with A_log and dt_bias learned per head, so 0 < gamma_t < 1 and a larger
    pre-activation decays the state faster;
  * beta_t = sigmoid(mean_s b[t, s]), so 0 < beta_t < 1.
"""
from __future__ import annotations

import numpy as np

from .gdn_ref import as_f64, gdn_head


def softplus(x):
    """ln(1 + e^x), evaluated without overflow."""
    return np.logaddexp(0.0, x)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def frame_gates(gate_a, gate_b, A_log: float, dt_bias: float):
    """gamma_t, beta_t of every frame of one head.  gate_a, gate_b: [T, S]
    per-token pre-activations; A_log, dt_bias: the head's parameters.
    Returns (gamma [T], beta [T]) in float64."""
    a = as_f64(gate_a).mean(axis=1)
    b = as_f64(gate_b).mean(axis=1)
    gamma = np.exp(-np.exp(float(A_log)) * softplus(a + float(dt_bias)))
    beta = sigmoid(b)
    return gamma, beta


def gdn_head_gated(q, k, v, gate_a, gate_b, A_log, dt_bias, state=None, key_scale: float = 1.0,
                   out_frames=None):
    """The frame-wise GDN forward of one head with its gates computed from
    activations (frame_gates) and its keys multiplied by key_scale.
    Returns (O, M_T, gamma, beta)."""
    gamma, beta = frame_gates(gate_a, gate_b, A_log, dt_bias)
    k = as_f64(k) * float(key_scale)
    O, M = gdn_head(q, k, v, gamma, beta, state, out_frames=out_frames)
    return O, M, gamma, beta
