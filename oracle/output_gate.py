"""fp64 oracle of the gated-retention output epilogue (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
use this module; the library never imports it and it shares no code with it.

What it computes (page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次",
section "路线二：Multi-Head Gated Retention", the paragraph after the state
recurrence): the multi-head output is normalised per head (GroupNorm, which
keeps the heads' scales from drifting apart) and then multiplied element by
element by the output gate swish(X W_G). The formula itself is not legible on
the page, so the plainest reading of those words is taken:

  for every (batch b, head h, position n):
      o       = out[b, h, n, :]                       (the head's dv values)
      mu      = mean(o),  var = mean((o - mu)^2)      (biased, as GroupNorm)
      z[j]    = (o[j] - mu) / sqrt(var + eps) * weight[h, j] + bias[h, j]
      y[j]    = swish(gate[b, h, n, j]) * z[j],       swish(x) = x / (1 + exp(-x))

i.e. GroupNorm with one group per head over the H*dv channels of a position,
an optional per-channel affine (weight 1 and bias 0 when absent), and the
SiLU/swish gate. The gate input X W_G is an argument: the projection itself
is outside the hot path. Everything is carried in float64; bf16 inputs (uint16
bit patterns) and float32 inputs are widened exactly.

Layouts: prefill out/gate [B, H, N, dv]; decode out/gate [B, H, dv];
weight/bias [H, dv]. The head axis is axis 1 in both.
"""
from __future__ import annotations

import numpy as np


def _widen(a: np.ndarray) -> np.ndarray:
    """float32 -> float64, or bf16 bit patterns (uint16) -> float64, exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError("unsupported dtype %s" % a.dtype)


def oracle_output_gate_f64(o, gate, weight=None, bias=None, eps: float = 1e-5) -> np.ndarray:
    """y = swish(gate) * GroupNorm_per_head(o) in float64 (see the module docstring).

    o: the retention output [B, H, N, dv] or [B, H, dv] (float64, float32 or
    bf16 bits); gate: same shape; weight, bias: [H, dv] or None.
    """
    x = _widen(o) if np.asarray(o).dtype != np.float64 else np.asarray(o)
    g = _widen(gate)
    if x.shape != g.shape:
        raise ValueError("o and gate shapes differ: %s vs %s" % (x.shape, g.shape))
    H, dv = x.shape[1], x.shape[-1]
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    z = (x - mu) / np.sqrt(var + eps)
    bshape = (1, H) + (1,) * (x.ndim - 3) + (dv,)
    if weight is not None:
        w = np.asarray(weight, dtype=np.float64)
        if w.shape != (H, dv):
            raise ValueError("weight must be [H, dv]")
        z = z * w.reshape(bshape)
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)
        if b.shape != (H, dv):
            raise ValueError("bias must be [H, dv]")
        z = z + b.reshape(bshape)
    swish = g / (1.0 + np.exp(-g))
    return swish * z
