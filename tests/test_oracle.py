"""Pins for the fp64 oracle: it is checked against things other than itself.

Every check below is fixed by the recurrence of the page "YOCO 完全拆解：
Decoder-Decoder 架构如何让 KV Cache 只存一次" (section "路线二：Multi-Head Gated
Retention": state decay by the head gate, key/value outer product, output from
the updated state; its unrolled form with the survival product of the gates) or
by plain mathematics (geometric series, causal linear attention, the RetNet
parallel form with a constant gate, linearity, independence of heads).
"""
import math
import os

import numpy as np
import pytest

from tests.chunk_form import brute_force_f64, chunk_form_f64, segment_form_f64
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_head(rng, N, dk, dv, lg_lo=-0.4, lg_hi=0.0, s0=True):
    q = rng.standard_normal((N, dk)).astype(np.float32)
    k = rng.standard_normal((N, dk)).astype(np.float32)
    v = rng.standard_normal((N, dv)).astype(np.float32)
    lg = rng.uniform(lg_lo, lg_hi, N).astype(np.float32)
    S0 = rng.standard_normal((dk, dv)).astype(np.float32) if s0 else None
    return q, k, v, lg, S0


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def test_golden_worked_example(oracle_lib):
    vals = {}
    with open(os.path.join(GOLDEN, "worked_example_dk2_dv3.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = [float(x) for x in rest]
    dk, dv = int(vals["dk"][0]), int(vals["dv"][0])
    N = len(vals["log_gamma"])
    q = np.array(vals["q"], np.float32).reshape(N, dk)
    k = np.array(vals["k"], np.float32).reshape(N, dk)
    v = np.array(vals["v"], np.float32).reshape(N, dv)
    lg = np.array(vals["log_gamma"], np.float32)
    s0 = np.array(vals["s0"], np.float32).reshape(dk, dv)
    out, S, _ = oracle_lib.oracle_prefill_f64(q, k, v, lg, s0)
    np.testing.assert_array_equal(out, np.array(vals["out"]).reshape(N, dv))
    np.testing.assert_array_equal(S, np.array(vals["s_final"]).reshape(dk, dv))


@pytest.mark.parametrize("N,dk,dv", [(1, 1, 1), (5, 3, 5), (23, 4, 2), (40, 3, 5)])
def test_brute_force_expansion(oracle_lib, N, dk, dv):
    rng = np.random.default_rng(7 + N)
    B, H = 2, 3
    qs, ks, vs, lgs, s0s = [], [], [], [], []
    for _ in range(B * H):
        q, k, v, lg, s0 = _rand_head(rng, N, dk, dv, lg_lo=-1.5)
        lg[rng.random(N) < 0.1] = -np.inf  # hard resets
        qs.append(q), ks.append(k), vs.append(v), lgs.append(lg), s0s.append(s0)
    q = np.stack(qs).reshape(B, H, N, dk)
    k = np.stack(ks).reshape(B, H, N, dk)
    v = np.stack(vs).reshape(B, H, N, dv)
    lg = np.stack(lgs).reshape(B, H, N)
    s0 = np.stack(s0s).reshape(B, H, dk, dv)
    out, S, _ = oracle_lib.oracle_prefill_f64(q, k, v, lg, s0)
    for x in range(B * H):
        b, h = divmod(x, H)
        o_ref, s_ref = brute_force_f64(q[b, h], k[b, h], v[b, h], lg[b, h], s0[b, h])
        assert _rel(out[b, h], o_ref) < 1e-12
        assert _rel(S[b, h], s_ref) < 1e-12


def test_gamma_one_is_causal_linear_attention(oracle_lib):
    rng = np.random.default_rng(11)
    N, dk, dv = 37, 6, 4
    q, k, v, _, s0 = _rand_head(rng, N, dk, dv)
    lg = np.zeros(N, np.float32)
    out, S, _ = oracle_lib.oracle_prefill_f64(q, k, v, lg, s0)
    Q, K, V, S0 = (x.astype(np.float64) for x in (q, k, v, s0))
    ref = np.tril(Q @ K.T) @ V + Q @ S0
    assert _rel(out, ref) < 1e-13
    assert _rel(S, S0 + K.T @ V) < 1e-13


def test_gamma_zero_keeps_only_current_token(oracle_lib):
    rng = np.random.default_rng(12)
    N, dk, dv = 19, 5, 7
    q, k, v, _, s0 = _rand_head(rng, N, dk, dv)
    lg = np.full(N, -np.inf, np.float32)
    out, S, _ = oracle_lib.oracle_prefill_f64(q, k, v, lg, s0)
    Q, K, V = (x.astype(np.float64) for x in (q, k, v))
    ref = np.sum(Q * K, axis=1)[:, None] * V
    assert _rel(out, ref) < 1e-15
    np.testing.assert_array_equal(S, np.outer(K[-1], V[-1]))


@pytest.mark.parametrize("gamma", [0.5, 0.9, 0.999])
def test_constant_gamma_retnet_parallel_form(oracle_lib, gamma):
    rng = np.random.default_rng(13)
    N, dk, dv = 50, 4, 6
    q, k, v, _, s0 = _rand_head(rng, N, dk, dv)
    lg = np.full(N, np.float32(math.log(gamma)), np.float32)
    out, S, _ = oracle_lib.oracle_prefill_f64(q, k, v, lg, s0)
    g = math.exp(float(lg[0]))
    n = np.arange(N)
    D = np.where(n[:, None] >= n[None, :], g ** (n[:, None] - n[None, :]).astype(np.float64), 0.0)
    Q, K, V, S0 = (x.astype(np.float64) for x in (q, k, v, s0))
    ref = ((Q @ K.T) * D) @ V + (g ** (n + 1))[:, None] * (Q @ S0)
    assert _rel(out, ref) < 1e-12
    s_ref = (g ** N) * S0 + K.T @ ((g ** (N - 1 - n))[:, None] * V)
    assert _rel(S, s_ref) < 1e-12


def test_scalar_geometric_series(oracle_lib):
    N = 200
    gamma_lg = np.float32(math.log(0.97))
    ones = np.ones((1, N, 1), np.float32)
    out, S, _ = oracle_lib.oracle_prefill_f64(ones, ones, ones, np.full((1, N), gamma_lg))
    g = math.exp(float(gamma_lg))
    ref = (1.0 - g ** (np.arange(N) + 1.0)) / (1.0 - g)
    assert _rel(out[0, :, 0], ref) < 1e-13
    assert abs(S[0, 0, 0] - ref[-1]) < 1e-12 * ref[-1]


@pytest.mark.parametrize("C", [1, 7, 16, 64, 500])
def test_chunk_form_equals_oracle(oracle_lib, C):
    rng = np.random.default_rng(21 + C)
    N, dk, dv = 500, 8, 12
    q, k, v, lg, s0 = _rand_head(rng, N, dk, dv, lg_lo=-0.3)
    out, S, _ = oracle_lib.oracle_prefill_f64(q, k, v, lg, s0)
    o_c, s_c = chunk_form_f64(q, k, v, lg, s0, C)
    assert _rel(o_c, out) < 1e-12
    assert _rel(s_c, S) < 1e-12


def test_chunk_form_with_log_gamma_floor_matches_hard_reset(oracle_lib):
    """exp(-inf) makes the chunk form produce NaN (-inf - -inf); a finite floor
    on the log-gate reproduces the gate-zero result to rounding."""
    rng = np.random.default_rng(31)
    N, dk, dv = 96, 4, 4
    q, k, v, lg, s0 = _rand_head(rng, N, dk, dv)
    lg[::5] = -np.inf
    out, S, _ = oracle_lib.oracle_prefill_f64(q, k, v, lg, s0)
    o_nan, _ = chunk_form_f64(q, k, v, lg, s0, 32)
    assert np.isnan(o_nan).any()
    o_c, s_c = chunk_form_f64(q, k, v, lg, s0, 32, floor=-80.0)
    assert _rel(o_c, out) < 1e-12
    assert _rel(s_c, S) < 1e-12


@pytest.mark.parametrize("seg_chunks,threshold", [(2, -88.0), (4, -20.0), (3, -5.0), (1, -1e30)])
def test_segment_split_equals_oracle(oracle_lib, seg_chunks, threshold):
    rng = np.random.default_rng(41)
    N, dk, dv, C = 700, 6, 10, 32
    q, k, v, lg, s0 = _rand_head(rng, N, dk, dv, lg_lo=-0.6)
    out, S, _ = oracle_lib.oracle_prefill_f64(q, k, v, lg, s0)
    o_s, s_s, corrected = segment_form_f64(q, k, v, lg, s0, C, seg_chunks, threshold)
    assert _rel(s_s, S) < 1e-12
    # dropped terms are below exp(threshold) times |q||S_in|
    tol = 1e-12 if threshold < -80 else 10.0 * math.exp(threshold)
    assert _rel(o_s, out) < tol
    assert corrected > 0


def test_split_resume_is_bitwise(oracle_lib):
    rng = np.random.default_rng(51)
    N1, N2, dk, dv = 61, 16, 5, 3
    q, k, v, lg, s0 = _rand_head(rng, N1 + N2, dk, dv)
    q, k, v, lg, s0 = q[None], k[None], v[None], lg[None], s0[None]
    out, S, _ = oracle_lib.oracle_prefill_f64(q, k, v, lg, s0)
    o1, s1, _ = oracle_lib.oracle_prefill_f64(q[:, :N1], k[:, :N1], v[:, :N1], lg[:, :N1], s0)
    o2, s2, _ = oracle_lib.oracle_prefill_f64(q[:, N1:], k[:, N1:], v[:, N1:], lg[:, N1:], s1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), out)
    np.testing.assert_array_equal(s2, S)
    # prefill(N1) followed by single-token decode steps
    st = s1.copy()
    for t in range(N1, N1 + N2):
        o = oracle_lib.oracle_decode_f64(q[:, t], k[:, t], v[:, t], lg[:, t], st)
        np.testing.assert_array_equal(o, out[:, t])
    np.testing.assert_array_equal(st, S)


def test_linearity_in_v_and_state(oracle_lib):
    rng = np.random.default_rng(61)
    N, dk, dv = 45, 4, 5
    q, k, _, lg, _ = _rand_head(rng, N, dk, dv)

    def dyadic(shape):  # multiples of 1/8 in [-8, 8): every combination below is exact
        return (rng.integers(-64, 64, shape) / 8.0).astype(np.float32)

    v1, v2, s01, s02 = dyadic((N, dv)), dyadic((N, dv)), dyadic((dk, dv)), dyadic((dk, dv))
    a, b = 0.75, -1.5
    o1, S1, _ = oracle_lib.oracle_prefill_f64(q, k, v1, lg, s01)
    o2, S2, _ = oracle_lib.oracle_prefill_f64(q, k, v2, lg, s02)
    o3, S3, _ = oracle_lib.oracle_prefill_f64(q, k, (a * v1 + b * v2).astype(np.float32), lg,
                                              (a * s01 + b * s02).astype(np.float32))
    assert _rel(o3, a * o1 + b * o2) < 1e-12
    assert _rel(S3, a * S1 + b * S2) < 1e-12
    qd = dyadic((N, dk))
    o5, _, _ = oracle_lib.oracle_prefill_f64(qd, k, v1, lg, s01)
    o4, _, _ = oracle_lib.oracle_prefill_f64((a * qd).astype(np.float32), k, v1, lg, s01)
    assert _rel(o4, a * o5) < 1e-13


def test_heads_are_independent(oracle_lib):
    rng = np.random.default_rng(71)
    B, H, N, dk, dv = 2, 4, 33, 3, 4
    q = rng.standard_normal((B, H, N, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, N, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, N, dv)).astype(np.float32)
    lg = rng.uniform(-0.5, 0, (B, H, N)).astype(np.float32)
    out, S, _ = oracle_lib.oracle_prefill_f64(q, k, v, lg)
    perm = rng.permutation(B * H)

    def p(x):
        return x.reshape((B * H,) + x.shape[2:])[perm].reshape(x.shape)

    out_p, S_p, _ = oracle_lib.oracle_prefill_f64(p(q), p(k), p(v), p(lg))
    np.testing.assert_array_equal(out_p, p(out))
    np.testing.assert_array_equal(S_p, p(S))


def test_bf16_inputs_are_widened_exactly(oracle_lib):
    rng = np.random.default_rng(81)
    N, dk, dv = 20, 8, 8
    q, k, v, lg, _ = _rand_head(rng, N, dk, dv, s0=False)
    qb, kb, vb = (f32_to_bf16_bits(x) for x in (q, k, v))
    o_b, S_b, _ = oracle_lib.oracle_prefill_f64(qb, kb, vb, lg)
    o_f, S_f, _ = oracle_lib.oracle_prefill_f64(*(bf16_bits_to_f32(x) for x in (qb, kb, vb)), lg)
    np.testing.assert_array_equal(o_b, o_f)
    np.testing.assert_array_equal(S_b, S_f)


def test_compare_statistics(oracle_lib):
    rng = np.random.default_rng(91)
    N, dk, dv = 30, 4, 4
    q, k, v, lg, s0 = _rand_head(rng, N, dk, dv)
    out, _, _ = oracle_lib.oracle_prefill_f64(q, k, v, lg, s0)
    cmp = out.astype(np.float32)
    cmp[3, 2] += 0.5
    _, _, stats = oracle_lib.oracle_prefill_f64(q, k, v, lg, s0, want_out=False, compare=cmp)
    assert stats.shape == (1, 2)
    assert abs(stats[0, 1] - np.max(np.abs(out))) == 0.0
    assert abs(stats[0, 0] - np.max(np.abs(cmp - out))) == 0.0


def test_three_b_state_size_arithmetic():
    # 13 Self-Decoder layers x 24 heads x (128 x 128) bf16 states is about 9.75 MiB
    # per request (page 1, section "用 3B 配置手算一遍"): the per-head state is
    # dk x dv and does not depend on the sequence length.
    from workloads import CONFIGS

    for name in ("prefill_32k", "prefill_512k", "prefill_1m", "decode_b256"):
        c = CONFIGS[name]
        assert (c["H"], c["dk"], c["dv"]) == (24, 128, 128)
    assert 13 * 24 * 128 * 128 * 2 == int(9.75 * 2 ** 20)
