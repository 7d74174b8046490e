"""Python entry points over the C ABI (argument marshalling only).

Tensors are torch tensors on a ROCm device; torch provides device memory and
the current stream, and every step of the computation runs in libgdn's HIP
kernels.  Names mirror include/gdn.h.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import GDN_BF16, GDN_F32, Shape, check, lib

_DT = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}


def _dtype_code(t: torch.dtype) -> int:
    if t not in _DT:
        raise TypeError(f"unsupported dtype {t}; expected float32 or bfloat16")
    return _DT[t]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, shape, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")


def shape_of(q: torch.Tensor) -> Shape:
    if q.dim() != 5:
        raise ValueError("q must be [B, H, T, S, D]")
    B, H, T, S, D = q.shape
    return Shape(B, H, T, S, D)


def set_fused(enabled: bool) -> bool:
    """gdn_set_fused: enable or disable the fused kernel for later calls
    (process-wide); returns the previous setting."""
    return bool(lib().gdn_set_fused(1 if enabled else 0))


def set_single_frame(enabled: bool) -> bool:
    """gdn_set_single_frame: enable or disable the single-frame kernels for
    later calls (process-wide); returns the previous setting."""
    return bool(lib().gdn_set_single_frame(1 if enabled else 0))


def workspace_bytes(B: int, H: int, T: int, S: int, D: int, in_dtype: torch.dtype) -> int:
    shp = Shape(B, H, T, S, D)
    return int(lib().gdn_workspace_bytes(ctypes.byref(shp), _dtype_code(in_dtype)))


def frame_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor,
              beta: torch.Tensor, state: Optional[torch.Tensor] = None,
              out_dtype: torch.dtype = torch.float32, *, out: Optional[torch.Tensor] = None,
              state_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
              key_scale: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Frame-wise GDN forward (gdn_frame_fwd; gdn_frame_fwd_ks when key_scale
    is given).

    q, k, v: [B, H, T, S, D] bf16 or f32; gamma, beta: [B, H, T] f32;
    state: [B, H, D, D] f32 or None (zeros).  Without key_scale, k is already
    scaled (by 1/sqrt(D*S) in the pages' setting); with it, the build runs on
    key_scale * k.
    Returns (out [B, H, T, S, D] out_dtype, state_out [B, H, D, D] f32).
    state_out may be the same tensor as state (in-place streaming)."""
    shp = shape_of(q)
    B, H, T, S, D = q.shape
    dev = q.device
    _need(q, "q", (B, H, T, S, D), None, dev)
    _need(k, "k", (B, H, T, S, D), q.dtype, dev)
    _need(v, "v", (B, H, T, S, D), q.dtype, dev)
    _need(gamma, "gamma", (B, H, T), torch.float32, dev)
    _need(beta, "beta", (B, H, T), torch.float32, dev)
    if state is not None:
        _need(state, "state", (B, H, D, D), torch.float32, dev)
    in_code, out_code = _dtype_code(q.dtype), _dtype_code(out_dtype)
    if out is None:
        out = torch.empty((B, H, T, S, D), dtype=out_dtype, device=dev)
    _need(out, "out", (B, H, T, S, D), out_dtype, dev)
    if state_out is None:
        state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    _need(state_out, "state_out", (B, H, D, D), torch.float32, dev)
    L = lib()
    wsb = int(L.gdn_workspace_bytes(ctypes.byref(shp), in_code))
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    if key_scale is None:
        st = L.gdn_frame_fwd(ctypes.byref(shp), in_code, out_code, _ptr(q), _ptr(k), _ptr(v),
                             _ptr(gamma), _ptr(beta), _ptr(state), _ptr(out), _ptr(state_out),
                             _ptr(workspace), workspace.numel(), _stream(dev))
        check(st, "gdn_frame_fwd")
    else:
        st = L.gdn_frame_fwd_ks(ctypes.byref(shp), in_code, out_code, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(gamma), _ptr(beta), _ptr(state), float(key_scale), _ptr(out),
                                _ptr(state_out), _ptr(workspace), workspace.numel(), _stream(dev))
        check(st, "gdn_frame_fwd_ks")
    return out, state_out


def frame_fwd_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate_a: torch.Tensor, gate_b: torch.Tensor,
                    A_log: torch.Tensor, dt_bias: torch.Tensor, state: Optional[torch.Tensor] = None,
                    key_scale: float = 1.0, out_dtype: torch.dtype = torch.float32, *,
                    workspace: Optional[torch.Tensor] = None):
    """Frame-wise GDN forward with its gates computed from activations
    (gdn_frame_fwd_gated): gamma_t = exp(-exp(A_log[h]) * softplus(mean_s
    gate_a + dt_bias[h])), beta_t = sigmoid(mean_s gate_b), keys multiplied
    by key_scale.  gate_a, gate_b: [B, H, T, S] f32; A_log, dt_bias: [H] f32.
    Returns (out, state_out, gamma [B, H, T], beta [B, H, T])."""
    shp = shape_of(q)
    B, H, T, S, D = q.shape
    dev = q.device
    _need(q, "q", (B, H, T, S, D), None, dev)
    _need(k, "k", (B, H, T, S, D), q.dtype, dev)
    _need(v, "v", (B, H, T, S, D), q.dtype, dev)
    _need(gate_a, "gate_a", (B, H, T, S), torch.float32, dev)
    _need(gate_b, "gate_b", (B, H, T, S), torch.float32, dev)
    _need(A_log, "A_log", (H,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H,), torch.float32, dev)
    if state is not None:
        _need(state, "state", (B, H, D, D), torch.float32, dev)
    out = torch.empty((B, H, T, S, D), dtype=out_dtype, device=dev)
    state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    gamma = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    beta = torch.empty_like(gamma)
    L = lib()
    in_code = _dtype_code(q.dtype)
    wsb = int(L.gdn_workspace_bytes(ctypes.byref(shp), in_code))
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    st = L.gdn_frame_fwd_gated(ctypes.byref(shp), in_code, _dtype_code(out_dtype), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(gate_a), _ptr(gate_b), _ptr(A_log), _ptr(dt_bias), _ptr(state),
                               float(key_scale), _ptr(out), _ptr(state_out), _ptr(gamma), _ptr(beta),
                               _ptr(workspace), workspace.numel(), _stream(dev))
    check(st, "gdn_frame_fwd_gated")
    return out, state_out, gamma, beta


def frame_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor,
              d_out: torch.Tensor, state: Optional[torch.Tensor] = None,
              d_state_out: Optional[torch.Tensor] = None, *,
              d_state_in: Optional[torch.Tensor] = None, key_scale: Optional[float] = None):
    """Backward pass of frame_fwd (gdn_frame_bwd; gdn_frame_bwd_ks when
    key_scale is given, dk then being the gradient with respect to the
    unscaled keys): gradients of <d_out, out> + <d_state_out, state_out>.

    q, k, v, d_out: [B, H, T, S, 128] bf16; gamma, beta: [B, H, T] f32;
    state, d_state_out: [B, H, 128, 128] f32 or None (zeros).  Returns
    (dq, dk, dv [B, H, T, S, 128] f32, dgamma, dbeta [B, H, T] f32,
    d_state_in [B, H, 128, 128] f32); d_state_in may be d_state_out."""
    shp = shape_of(q)
    B, H, T, S, D = q.shape
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (d_out, "d_out")):
        _need(t, name, (B, H, T, S, D), torch.bfloat16, dev)
    _need(gamma, "gamma", (B, H, T), torch.float32, dev)
    _need(beta, "beta", (B, H, T), torch.float32, dev)
    for t, name in ((state, "state"), (d_state_out, "d_state_out")):
        if t is not None:
            _need(t, name, (B, H, D, D), torch.float32, dev)
    grads = [torch.empty((B, H, T, S, D), dtype=torch.float32, device=dev) for _ in range(3)]
    dgamma = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dbeta = torch.empty_like(dgamma)
    if d_state_in is None:
        d_state_in = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    _need(d_state_in, "d_state_in", (B, H, D, D), torch.float32, dev)
    L = lib()
    wsb = int(L.gdn_bwd_workspace_bytes(ctypes.byref(shp), GDN_BF16))
    workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    tail = (_ptr(d_out), _ptr(d_state_out), _ptr(grads[0]), _ptr(grads[1]), _ptr(grads[2]), _ptr(dgamma),
            _ptr(dbeta), _ptr(d_state_in), _ptr(workspace), wsb, _stream(dev))
    head = (ctypes.byref(shp), GDN_BF16, _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta), _ptr(state))
    if key_scale is None:
        check(L.gdn_frame_bwd(*head, *tail), "gdn_frame_bwd")
    else:
        check(L.gdn_frame_bwd_ks(*head, float(key_scale), *tail), "gdn_frame_bwd_ks")
    return grads[0], grads[1], grads[2], dgamma, dbeta, d_state_in


def build_maps(k: torch.Tensor, v: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Stage 1 (gdn_build_maps): G_t = K_t^T K_t and U_t = V_t^T K_t, [B,H,T,D,D] f32."""
    shp = shape_of(k)
    B, H, T, S, D = k.shape
    dev = k.device
    _need(k, "k", (B, H, T, S, D), None, dev)
    _need(v, "v", (B, H, T, S, D), k.dtype, dev)
    G = torch.empty((B, H, T, D, D), dtype=torch.float32, device=dev)
    U = torch.empty_like(G)
    st = lib().gdn_build_maps(ctypes.byref(shp), _dtype_code(k.dtype), _ptr(k), _ptr(v), _ptr(G),
                              _ptr(U), _stream(dev))
    check(st, "gdn_build_maps")
    return G, U


def state_pass(G: torch.Tensor, U: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor,
               state: Optional[torch.Tensor] = None, keep_all: bool = True):
    """Stage 2 (gdn_state_pass): returns (M_all [B,H,T,D,D] or None, state_out [B,H,D,D])."""
    B, H, T, D, _ = G.shape
    dev = G.device
    shp = Shape(B, H, T, 1, D)
    _need(G, "G", (B, H, T, D, D), torch.float32, dev)
    _need(U, "U", (B, H, T, D, D), torch.float32, dev)
    _need(gamma, "gamma", (B, H, T), torch.float32, dev)
    _need(beta, "beta", (B, H, T), torch.float32, dev)
    if state is not None:
        _need(state, "state", (B, H, D, D), torch.float32, dev)
    M_all = torch.empty_like(G) if keep_all else None
    state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    st = lib().gdn_state_pass(ctypes.byref(shp), _ptr(G), _ptr(U), _ptr(gamma), _ptr(beta),
                              _ptr(state), _ptr(M_all), _ptr(state_out), _stream(dev))
    check(st, "gdn_state_pass")
    return M_all, state_out


def output(q: torch.Tensor, M_all: torch.Tensor, out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Stage 3 (gdn_output): O_t = Q_t M_t^T."""
    shp = shape_of(q)
    B, H, T, S, D = q.shape
    dev = q.device
    _need(q, "q", (B, H, T, S, D), None, dev)
    _need(M_all, "M_all", (B, H, T, D, D), torch.float32, dev)
    out = torch.empty((B, H, T, S, D), dtype=out_dtype, device=dev)
    st = lib().gdn_output(ctypes.byref(shp), _dtype_code(q.dtype), _dtype_code(out_dtype), _ptr(q),
                          _ptr(M_all), _ptr(out), _stream(dev))
    check(st, "gdn_output")
    return out


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sink: int, first_chunk: int, chunk: int,
             window: int, *, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None, want_lse: bool = True):
    """Softmax attention with attention sinks and a local temporal window
    (gdn_attn_fwd, include/gdn_attn.h).

    q, k, v: [B, H, T, S, 128] bf16.  A query of generation chunk c (chunk 0:
    the first `first_chunk` frames, then `chunk` frames each) sees the tokens
    of chunks c - window + 1 .. c and of the first `sink` frames up to chunk c.
    Returns (out [B, H, T, S, 128] f32, lse [B, H, T, S] f32 or None)."""
    shp = shape_of(q)
    B, H, T, S, D = q.shape
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, (B, H, T, S, D), torch.bfloat16, dev)
    if out is None:
        out = torch.empty((B, H, T, S, D), dtype=torch.float32, device=dev)
    _need(out, "out", (B, H, T, S, D), torch.float32, dev)
    if want_lse and lse is None:
        lse = torch.empty((B, H, T, S), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (B, H, T, S), torch.float32, dev)
    lay = _lib.AttnLayout(int(sink), int(first_chunk), int(chunk), int(window))
    st = lib().gdn_attn_fwd(ctypes.byref(shp), GDN_BF16, ctypes.byref(lay), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                            _ptr(lse), _stream(dev))
    check(st, "gdn_attn_fwd")
    return out, lse
