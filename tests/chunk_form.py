"""fp64 numpy evaluations of the chunkwise and segment-split forms of gated retention.

These are the re-associations the HIP kernels implement. They live with the
tests (never in the library) and are checked against the fp64 oracle, so the
algebra is validated independently of any kernel.

Chunkwise form (page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次",
section "Prefill 与 Decode 为什么使用两种计算形态"): for a chunk starting at
position a, with beta_j the inclusive running sum of log-gates inside the chunk,
  out[a+j] = sum_{l<=j} exp(beta_j - beta_l) (q_{a+j}.k_{a+l}) v_{a+l}
             + exp(beta_j) q_{a+j} S_{a-1}
  S_end    = exp(beta_last) S_{a-1} + sum_l exp(beta_last - beta_l) k_{a+l}^T v_{a+l}
The page states this is exact, only associated differently; the chunk size is a
tuning knob, not part of the result.
"""
from __future__ import annotations

import numpy as np


def chunk_form_f64(q, k, v, lg, s0, C, floor=None):
    """One head. q,k [N,dk], v [N,dv], lg [N] (float64), s0 [dk,dv] or None."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    lg = np.asarray(lg, np.float64)
    if floor is not None:
        lg = np.maximum(lg, floor)
    N, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if s0 is None else np.array(s0, np.float64)
    out = np.empty((N, dv))
    for a in range(0, N, C):
        e = min(a + C, N)
        beta = np.cumsum(lg[a:e])
        n = e - a
        causal = np.tril(np.ones((n, n), dtype=bool))
        with np.errstate(invalid="ignore", over="ignore"):
            diff = beta[:, None] - beta[None, :]
        decay = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
        qc, kc, vc = q[a:e], k[a:e], v[a:e]
        out[a:e] = ((qc @ kc.T) * decay) @ vc + np.exp(beta)[:, None] * (qc @ S)
        g = beta[-1]
        with np.errstate(invalid="ignore"):
            S = np.exp(g) * S + kc.T @ (np.exp(g - beta)[:, None] * vc)
    return out, S


def segment_form_f64(q, k, v, lg, s0, C, seg_chunks, threshold):
    """Segment-split evaluation (one head), the decomposition the prefill uses
    to run several parts of one sequence at once.

    The sequence is cut into segments of ``seg_chunks`` chunks. Every segment
    except the first runs from a zero state and yields its local output, its
    local end state and its total log-decay G. The states are then chained:
    S_end(p) = exp(G_p) S_end(p-1) + S_loc(p). The incoming state adds
    exp(B_n) q_n S_in to each output of the segment, where B_n is the running
    log-decay from the segment start; that term is kept only on the leading
    whole chunks of the segment until the running sum at a chunk end drops
    below ``threshold`` (log-gates are <= 0, so B_n only decreases).
    Returns (out, S_final, corrected_positions).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    lg = np.asarray(lg, np.float64)
    N, dk = q.shape
    dv = v.shape[1]
    L = seg_chunks * C
    out = np.empty((N, dv))
    S_prev = np.zeros((dk, dv)) if s0 is None else np.array(s0, np.float64)
    corrected = 0
    for a in range(0, N, L):
        e = min(a + L, N)
        if a == 0:
            o, S_prev = chunk_form_f64(q[a:e], k[a:e], v[a:e], lg[a:e], S_prev, C)
            out[a:e] = o
            continue
        o_loc, s_loc = chunk_form_f64(q[a:e], k[a:e], v[a:e], lg[a:e], None, C)
        B = np.cumsum(lg[a:e])
        # leading whole chunks whose end still has B >= threshold, plus the one
        # where it first drops below (its earlier rows may still need the term)
        m = 0
        n_seg = e - a
        while m * C < n_seg:
            m += 1
            if B[min(m * C, n_seg) - 1] < threshold:
                break
        h = min(m * C, n_seg)
        o_loc[:h] += np.exp(B[:h])[:, None] * (q[a:a + h] @ S_prev)
        corrected += h
        out[a:e] = o_loc
        S_prev = np.exp(B[-1]) * S_prev + s_loc
    return out, S_prev, corrected


def brute_force_f64(q, k, v, lg, s0=None):
    """Unrolled recurrence, O(N^2) (one head): the survival product of the gates
    strictly after m up to n multiplies token m's contribution to output n."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.exp(np.asarray(lg, np.float64))
    N, dk = q.shape
    dv = v.shape[1]
    out = np.zeros((N, dv))
    for n in range(N):
        for m in range(n + 1):
            surv = 1.0
            for t in range(m + 1, n + 1):
                surv *= g[t]
            out[n] += surv * float(q[n] @ k[m]) * v[m]
        if s0 is not None:
            surv = 1.0
            for t in range(0, n + 1):
                surv *= g[t]
            out[n] += surv * (q[n] @ np.asarray(s0, np.float64))
    S = np.zeros((dk, dv))
    for m in range(N):
        surv = 1.0
        for t in range(m + 1, N):
            surv *= g[t]
        S += surv * np.outer(k[m], v[m])
    if s0 is not None:
        surv = 1.0
        for t in range(N):
            surv *= g[t]
        S += surv * np.asarray(s0, np.float64)
    return out, S
