"""fp64 oracle of the Cross-Decoder's decode attention over the shared global
KV cache (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
use this module; the library never imports it and it shares no code with it.

What it computes (page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次",
sections "增量生成时究竟追加什么" and "接入推理引擎时的四个关键点"): at a decode
step every Cross-Decoder layer forms its own query for the new token and
attends over the one global cache of keys and values of all positions so far
(the new token's included); with GQA the query heads outnumber the KV heads
and groups of query heads share one K/V head (the 3B configuration: 24 query
heads, 8 KV heads, three per KV head). Rotary position terms are applied to
queries and keys before they reach the cache and this step, so here:

  for every sequence b and query head h, with g = h // (Hq / Hkv) its KV head:
      s[t]   = scale * sum_j q[b,h,j] * K[b,g,t,j]     for t < length[b]
      p      = softmax(s)                               (over t < length[b])
      out[b,h,:] = sum_t p[t] * V[b,g,t,:]

Readings: the grouping is consecutive (query heads h = 3g, 3g+1, 3g+2 share KV
head g, as torch's repeat_interleave / enable_gqa), and the scale is an
argument (d^-1/2 by default, the usual dot-product attention scale).
Everything is carried in float64; bf16 (uint16 bit patterns) and float32
inputs are widened exactly.

Layouts: q [B, Hq, d]; K, V [B, Hkv, Lmax, d]; length [B] (int) or None (all
Lmax); out [B, Hq, d].
"""
from __future__ import annotations

import numpy as np


def _widen(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def oracle_cross_attention_f64(q, k_cache, v_cache, length=None, scale=None) -> np.ndarray:
    """Decode attention of every query head over its KV head's cache (float64)."""
    qd, kd, vd = _widen(q), _widen(k_cache), _widen(v_cache)
    B, Hq, d = qd.shape
    _, Hkv, Lmax, dk = kd.shape
    if dk != d or vd.shape[:3] != (B, Hkv, Lmax):
        raise ValueError("shape mismatch")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lens = np.full(B, Lmax, dtype=np.int64) if length is None else np.asarray(length, np.int64)
    out = np.zeros((B, Hq, vd.shape[3]), dtype=np.float64)
    for b in range(B):
        n = int(lens[b])
        if not 1 <= n <= Lmax:
            raise ValueError("length must be in [1, Lmax]")
        for h in range(Hq):
            g = h // group
            s = scale * (kd[b, g, :n] @ qd[b, h])
            s = s - s.max()
            p = np.exp(s)
            p /= p.sum()
            out[b, h] = p @ vd[b, g, :n]
    return out
