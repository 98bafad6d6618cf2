"""Pins of the sliding-window-attention oracle to facts outside it: torch's
scaled_dot_product_attention with an explicit window mask (float64, CPU),
explicit loops on tiny inputs, the closed forms of a one-position window and
of constant keys (plain window averages), and a decode loop that must retrace
the prefill rows and leave the ring the prefill leaves."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle_swa_decode_f64, oracle_swa_prefill_f64, oracle_swa_ring_f64


def sdpa_window(q, k, v, window, scale=None):
    """torch reference: keys repeated per query-head group, boolean window mask."""
    qt, kt, vt = (torch.from_numpy(np.asarray(a, np.float64)) for a in (q, k, v))
    G = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(G, dim=1)
    vt = vt.repeat_interleave(G, dim=1)
    N = qt.shape[2]
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    mask = (j <= i) & (j > i - window)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                            scale=scale).numpy()


@pytest.mark.parametrize("N,window,Hq,Hkv", [(50, 8, 2, 2), (70, 16, 4, 2), (40, 100, 3, 1),
                                             (33, 1, 2, 1), (64, 64, 2, 2)])
def test_prefill_matches_torch_window_mask(N, window, Hq, Hkv):
    rng = np.random.default_rng(N + window)
    d = 16
    q = rng.standard_normal((2, Hq, N, d))
    k = rng.standard_normal((2, Hkv, N, d))
    v = rng.standard_normal((2, Hkv, N, d))
    got = oracle_swa_prefill_f64(q, k, v, window)
    np.testing.assert_allclose(got, sdpa_window(q, k, v, window), rtol=1e-10, atol=1e-12)


def test_prefill_selected_rows_match_torch_window_mask():
    """The rows option (used where only sampled outputs of a long prompt are
    checked): every listed row equals the same row of torch's masked attention,
    whether q holds the whole prompt or only the listed rows."""
    rng = np.random.default_rng(77)
    N, d, C, Hq, Hkv = 90, 8, 16, 4, 2
    q = rng.standard_normal((2, Hq, N, d))
    k = rng.standard_normal((2, Hkv, N, d))
    v = rng.standard_normal((2, Hkv, N, d))
    rows = np.array([0, 1, 15, 16, 17, 50, 89])
    ref = sdpa_window(q, k, v, C)[:, :, rows]
    np.testing.assert_allclose(oracle_swa_prefill_f64(q, k, v, C, rows=rows), ref,
                               rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(oracle_swa_prefill_f64(q[:, :, rows], k, v, C, rows=rows), ref,
                               rtol=1e-10, atol=1e-12)
    with pytest.raises(ValueError):
        oracle_swa_prefill_f64(q, k, v, C, rows=[N])
    with pytest.raises(ValueError):
        oracle_swa_prefill_f64(q[:, :, :5], k, v, C, rows=rows)


def test_prefill_explicit_loops_tiny():
    rng = np.random.default_rng(5)
    N, d, C = 9, 3, 4
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    got = oracle_swa_prefill_f64(q, k, v, C, scale=0.7)
    for i in range(N):
        js = range(max(0, i - C + 1), i + 1)
        w = [math.exp(0.7 * sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d))) for j in js]
        ref = [sum(wj * v[0, 0, j, t] for wj, j in zip(w, js)) / sum(w) for t in range(d)]
        np.testing.assert_allclose(got[0, 0, i], ref, rtol=1e-12)


def test_window_one_returns_own_value():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 4, 20, 8))
    k = rng.standard_normal((1, 2, 20, 8))
    v = rng.standard_normal((1, 2, 20, 8))
    got = oracle_swa_prefill_f64(q, k, v, 1)
    np.testing.assert_array_equal(got[0, 0], v[0, 0])
    np.testing.assert_array_equal(got[0, 3], v[0, 1])   # query head 3 reads KV head 1


def test_constant_keys_average_the_window():
    rng = np.random.default_rng(7)
    N, C, d = 40, 6, 5
    q = rng.standard_normal((1, 1, N, d))
    k = np.ones((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    got = oracle_swa_prefill_f64(q, k, v, C)
    cs = np.concatenate([np.zeros((1, d)), np.cumsum(v[0, 0], axis=0)])
    for i in range(N):
        lo = max(0, i - C + 1)
        np.testing.assert_allclose(got[0, 0, i], (cs[i + 1] - cs[lo]) / (i + 1 - lo), rtol=1e-12)


@pytest.mark.parametrize("N,C", [(5, 8), (21, 8), (16, 8)])
def test_decode_steps_retrace_prefill_and_ring(N, C):
    rng = np.random.default_rng(N * C)
    B, Hq, Hkv, d = 2, 4, 2, 8
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    ref = oracle_swa_prefill_f64(q, k, v, C)
    rk = np.zeros((B, Hkv, C, d))
    rv = np.zeros((B, Hkv, C, d))
    for t in range(N):
        out, rk, rv = oracle_swa_decode_f64(q[:, :, t], k[:, :, t], v[:, :, t], rk, rv,
                                            np.full(B, t))
        np.testing.assert_allclose(out, ref[:, :, t], rtol=1e-11, atol=1e-13)
    wk, wv = oracle_swa_ring_f64(k, v, C)
    np.testing.assert_array_equal(rk, wk)
    np.testing.assert_array_equal(rv, wv)


def test_decode_sequences_at_different_positions():
    # sequence 0 at position 3 (ring partly filled), sequence 1 at 11 (wrapped)
    rng = np.random.default_rng(9)
    C, d = 8, 4
    q = rng.standard_normal((2, 1, 12, d))
    k = rng.standard_normal((2, 1, 12, d))
    v = rng.standard_normal((2, 1, 12, d))
    ref = oracle_swa_prefill_f64(q, k, v, C)
    rk0, rv0 = oracle_swa_ring_f64(k[:, :, :3], v[:, :, :3], C)
    rk1, rv1 = oracle_swa_ring_f64(k[:, :, :11], v[:, :, :11], C)
    rk = np.stack([rk0[0], rk1[1]])
    rv = np.stack([rv0[0], rv1[1]])
    pos = np.array([3, 11])
    out, _, _ = oracle_swa_decode_f64(q[[0, 1], :, pos], k[[0, 1], :, pos], v[[0, 1], :, pos],
                                      rk, rv, pos)
    np.testing.assert_allclose(out[0], ref[0, :, 3], rtol=1e-11)
    np.testing.assert_allclose(out[1], ref[1, :, 11], rtol=1e-11)
