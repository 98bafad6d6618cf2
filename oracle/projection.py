"""fp64 oracle of the key and log-gate projections that feed gated retention,
with the key scaling and the gate's temperature applied in the projection's
epilogue (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
use this module; the library never imports it and it shares no code with it.

What it computes (page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次"):
section "路线二：Multi-Head Gated Retention" has each head project the hidden
state of position n to its key K_n and to a data-dependent gate
gamma_n = sigmoid(X_n W_gamma)^(1/tau), whose temperature tau keeps gamma near
1; section "单 token Decode 的实现骨架" adds that the official code divides the
gate's log value by 16 and scales K by d_h^(-1/2). The retention consumes
the log-gate l = log gamma, so for token m = (b, n), head h, key channel c:

    K[b, h, n, c] = key_scale * sum_d x[b, n, d] * W_K[h * dk + c, d]
    u[b, h, n]    = sum_d x[b, n, d] * W_gamma[h, d]
    l[b, h, n]    = log(sigmoid(u)) / tau = (min(u, 0) - log(1 + exp(-|u|))) / tau

(the second form of log sigmoid is the same function written so that no
exponential overflows). Readings: the weights are stored as linear-layer
rows (one row of D weights per output channel), there is no bias, key_scale
and tau are arguments (d_h^-1/2 and 16 in the pages' model).

Layouts: x [B, N, D] (bf16 as uint16 bit patterns, or float); W_K [H*dk, D];
W_gamma [H, D] or None. Returns K [B, H, N, dk] and l [B, H, N] (None
without W_gamma), both float64.
"""
from __future__ import annotations

import numpy as np


def _widen(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def log_sigmoid_f64(u):
    """log(sigmoid(u)) = -log(1 + exp(-u)), evaluated without overflow."""
    u = np.asarray(u, dtype=np.float64)
    return np.minimum(u, 0.0) - np.log1p(np.exp(-np.abs(u)))


def oracle_head_projection_f64(x, w_key, w_gamma=None, key_scale=1.0, temperature=16.0, H=None):
    """Head-major key projection (times key_scale) and, when w_gamma is given,
    the log-gate log(sigmoid(x W_gamma)) / temperature of every head."""
    xd = _widen(x)
    wk = _widen(w_key)
    B, N, D = xd.shape
    J, Dw = wk.shape
    if Dw != D:
        raise ValueError("weight width must equal the hidden size")
    if H is None:
        if w_gamma is None:
            raise ValueError("H is needed without W_gamma")
        H = _widen(w_gamma).shape[0]
    if J % H != 0:
        raise ValueError("key rows must be H * dk")
    dk = J // H
    proj = xd.reshape(B * N, D) @ wk.T                                # [B*N, H*dk]
    k = key_scale * proj.reshape(B, N, H, dk).transpose(0, 2, 1, 3)  # [B, H, N, dk]
    lg = None
    if w_gamma is not None:
        wg = _widen(w_gamma)
        if wg.shape != (H, D):
            raise ValueError("W_gamma must be [H, D]")
        u = (xd.reshape(B * N, D) @ wg.T).reshape(B, N, H).transpose(0, 2, 1)  # [B, H, N]
        lg = log_sigmoid_f64(u) / temperature
    return np.ascontiguousarray(k), None if lg is None else np.ascontiguousarray(lg)
