"""Pins of the projection oracle (key scaling and log-gate epilogue) to facts
that do not come from the oracle itself: explicit sums and the textbook
sigmoid on tiny inputs, the identity sigmoid(u) + sigmoid(-u) = 1, exact
special values, and layout-revealing weights (identity and one-hot rows)."""
import math

import numpy as np
import pytest

from oracle import log_sigmoid_f64, oracle_head_projection_f64
from workloads import f32_to_bf16_bits


def brute(x, wk, wg, scale, tau, H):
    """Python loops: K by explicit sums, the gate by log of 1 / (1 + e^-u)."""
    B, N, D = x.shape
    dk = wk.shape[0] // H
    K = np.zeros((B, H, N, dk))
    L = np.zeros((B, H, N))
    for b in range(B):
        for n in range(N):
            for h in range(H):
                for c in range(dk):
                    K[b, h, n, c] = scale * sum(float(x[b, n, d]) * float(wk[h * dk + c, d])
                                                for d in range(D))
                u = sum(float(x[b, n, d]) * float(wg[h, d]) for d in range(D))
                L[b, h, n] = math.log(1.0 / (1.0 + math.exp(-u))) / tau
    return K, L


def test_brute_force_tiny():
    rng = np.random.default_rng(1)
    B, N, D, H, dk = 2, 3, 5, 2, 3
    x = rng.standard_normal((B, N, D))
    wk = rng.standard_normal((H * dk, D))
    wg = rng.standard_normal((H, D))
    K, L = oracle_head_projection_f64(x, wk, wg, key_scale=0.37, temperature=16.0)
    Kb, Lb = brute(x, wk, wg, 0.37, 16.0, H)
    np.testing.assert_allclose(K, Kb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=1e-12, atol=1e-14)


def test_sigmoid_complement_identity():
    # sigmoid(u) + sigmoid(-u) = 1: gamma^tau of a gate plus that of the negated
    # gate weights is 1 for every head and position.
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 7, 16))
    wk = rng.standard_normal((4 * 2, 16))
    wg = 0.5 * rng.standard_normal((4, 16))
    tau = 16.0
    _, Lp = oracle_head_projection_f64(x, wk, wg, temperature=tau)
    _, Lm = oracle_head_projection_f64(x, wk, -wg, temperature=tau)
    np.testing.assert_allclose(np.exp(tau * Lp) + np.exp(tau * Lm), 1.0, rtol=0, atol=1e-13)


def test_zero_logit_gives_half():
    x = np.ones((1, 2, 8))
    _, L = oracle_head_projection_f64(x, np.zeros((3 * 4, 8)), np.zeros((3, 8)), temperature=16.0)
    np.testing.assert_allclose(L, -math.log(2.0) / 16.0, rtol=0, atol=1e-16)


@pytest.mark.parametrize("u", [800.0, -800.0, 40.0, -40.0])
def test_extreme_logits_finite(u):
    x = np.full((1, 1, 1), u)
    _, L = oracle_head_projection_f64(x, np.zeros((1, 1)), np.ones((1, 1)), temperature=16.0)
    assert np.isfinite(L).all()
    # log sigmoid(u) -> u for u -> -inf and -> -e^-u for u -> +inf
    want = (u - math.exp(u)) / 16.0 if u < 0 else -math.exp(-u) / 16.0
    np.testing.assert_allclose(L[0, 0, 0], want, rtol=1e-12, atol=1e-300)


def test_identity_weights_reveal_head_major_layout():
    rng = np.random.default_rng(3)
    B, N, H, dk = 2, 5, 3, 4
    D = H * dk
    x = rng.standard_normal((B, N, D))
    K, L = oracle_head_projection_f64(x, np.eye(D), None, key_scale=0.5, H=H)
    assert L is None
    for b in range(B):
        for h in range(H):
            for n in range(N):
                np.testing.assert_array_equal(K[b, h, n], 0.5 * x[b, n, h * dk:(h + 1) * dk])


def test_one_hot_gate_rows_select_hidden_channels():
    rng = np.random.default_rng(4)
    B, N, D, H = 2, 6, 9, 3
    x = rng.standard_normal((B, N, D))
    wg = np.zeros((H, D))
    for h in range(H):
        wg[h, 2 * h + 1] = 1.0
    _, L = oracle_head_projection_f64(x, np.zeros((H, D)), wg, temperature=4.0)
    for h in range(H):
        u = x[:, :, 2 * h + 1]
        np.testing.assert_allclose(L[:, h, :], -np.log1p(np.exp(-u)) / 4.0, rtol=1e-13)


def test_bf16_bits_widened_exactly():
    x = np.array([[[1.0, -2.0, 0.5]]], dtype=np.float32)
    w = np.array([[1.0, 1.0, 1.0]], dtype=np.float32)
    K, _ = oracle_head_projection_f64(f32_to_bf16_bits(x), f32_to_bf16_bits(w), None, H=1)
    assert K[0, 0, 0, 0] == -0.5


def test_log_sigmoid_matches_definition_midrange():
    u = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(log_sigmoid_f64(u), [math.log(1 / (1 + math.exp(-t))) for t in u],
                               rtol=1e-12, atol=2e-16)
