"""fp64 oracle of the sliding-window-attention Self-Decoder mixer: prefill
over a prompt and one decode step over a ring buffer of the last C keys and
values (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
use this module; the library never imports it and it shares no code with it.

What it computes (page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次",
section "路线一：滑动窗口注意力"): position i attends only to the most recent C
positions, i.e. softmax attention with the causal window mask that admits
j in [i - C + 1, i]; while decoding position n a layer keeps only the keys and
values of [n - C + 1, n], overwriting the oldest in a ring; the paper's runs
use C = 1024. Section "Prefill 的实现骨架" has the prefill leave the last C
keys and values of each layer in a fixed buffer for decoding. So, per
sequence b, query head h and its KV head g = h // (Hq / Hkv):

    out[b,h,i,:] = sum_j p_j v[b,g,j,:],  p = softmax_j(scale * q[b,h,i,:] . k[b,g,j,:])
                   over max(0, i - C + 1) <= j <= i

Readings: heads are grouped consecutively as in the Cross-Decoder (Hq = Hkv
is plain multi-head attention); the scale is an argument, d^-1/2 by default;
rotary position terms are applied to q and k before this step; ring slot of
position p is p mod C. The window admits C positions, the current included.

Layouts: q [B, Hq, N, d]; k, v [B, Hkv, N, d]; ring buffers [B, Hkv, C, d];
bf16 inputs are uint16 bit patterns (widened exactly), floats are used as is.
"""
from __future__ import annotations

import numpy as np


def _widen(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _attend(qv, ks, vs, scale):
    """softmax(scale * ks @ qv) @ vs for one query vector (float64)."""
    s = scale * (ks @ qv)
    s = s - s.max()
    p = np.exp(s)
    return (p / p.sum()) @ vs


def oracle_swa_prefill_f64(q, k, v, window, scale=None, rows=None):
    """Sliding-window causal attention of every query position (float64), one
    query row at a time over the keys of its own window.

    rows: optional 1-D sequence of query positions; then only those rows are
    computed (each exactly as above) and out is [B, Hq, len(rows), d], row r
    of it being position rows[r]. q may then hold just those rows
    ([B, Hq, len(rows), d]) or the whole prompt ([B, Hq, N, d])."""
    qd, kd, vd = _widen(q), _widen(k), _widen(v)
    B, Hq, Nq, d = qd.shape
    _, Hkv, N, dk = kd.shape
    if dk != d or vd.shape[:3] != (B, Hkv, N):
        raise ValueError("shape mismatch")
    if Hq % Hkv != 0 or window < 1:
        raise ValueError("Hq must be a multiple of Hkv and the window positive")
    if rows is None:
        pos = np.arange(N)
        if Nq != N:
            raise ValueError("shape mismatch")
        qrow = pos
    else:
        pos = np.asarray(rows, dtype=np.int64).reshape(-1)
        if pos.size and (pos.min() < 0 or pos.max() >= N):
            raise ValueError("rows out of range")
        if Nq == pos.size:
            qrow = np.arange(pos.size)
        elif Nq == N:
            qrow = pos
        else:
            raise ValueError("q must hold the listed rows or the whole prompt")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, pos.size, vd.shape[3]), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r in range(pos.size):
                i = int(pos[r])
                j0 = max(0, i - window + 1)
                out[b, h, r] = _attend(qd[b, h, qrow[r]], kd[b, g, j0:i + 1], vd[b, g, j0:i + 1],
                                       scale)
    return out


def oracle_swa_ring_f64(k, v, window):
    """The ring buffers a prefill of N positions leaves: slot p mod C holds
    position p for the last min(N, C) positions; other slots are zero."""
    kd, vd = _widen(k), _widen(v)
    B, Hkv, N, d = kd.shape
    rk = np.zeros((B, Hkv, window, d))
    rv = np.zeros((B, Hkv, window, vd.shape[3]))
    for p in range(max(0, N - window), N):
        rk[:, :, p % window] = kd[:, :, p]
        rv[:, :, p % window] = vd[:, :, p]
    return rk, rv


def oracle_swa_decode_f64(q, k_new, v_new, ring_k, ring_v, positions, scale=None):
    """One decode step: write the new token's key and value (position
    positions[b]) into ring slot positions[b] mod C, then attend each query
    head over the slots that hold positions max(0, pos - C + 1) .. pos.
    Returns (out [B, Hq, d], ring_k, ring_v) with the rings updated (copies)."""
    qd, kn, vn = _widen(q), _widen(k_new), _widen(v_new)
    rk, rv = _widen(ring_k).copy(), _widen(ring_v).copy()
    B, Hq, d = qd.shape
    _, Hkv, C, _ = rk.shape
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, rv.shape[3]))
    for b in range(B):
        pos = int(positions[b])
        if pos < 0:
            raise ValueError("positions must be >= 0")
        rk[b, :, pos % C] = kn[b]
        rv[b, :, pos % C] = vn[b]
        valid = [p % C for p in range(max(0, pos - C + 1), pos + 1)]
        for h in range(Hq):
            g = h // G
            out[b, h] = _attend(qd[b, h], rk[b, g, valid], rv[b, g, valid], scale)
    return out, rk, rv
