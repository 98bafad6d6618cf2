"""Pins for the fp64 Cross-Decoder decode-attention oracle.

The definition follows the page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV
Cache 只存一次" (sections "增量生成时究竟追加什么" and "接入推理引擎时的四个关键点":
every Cross layer's query for the new token attends over the single global
K/V cache; with GQA, groups of query heads share one KV head). It is checked
against torch's scaled_dot_product_attention in float64 (a library routine),
a hand-worked example and closed forms.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle_cross_attention_f64


def _rand(rng, B, Hq, Hkv, L, d):
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, L, d))
    v = rng.standard_normal((B, Hkv, L, d))
    return q, k, v


def test_worked_example():
    # scale 1, q = [1, 0]: scores are the first key components [0, ln 3], so the
    # softmax weights are [1/4, 3/4] and out = V^T p = [1, -1].
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[[0.0, 5.0], [math.log(3.0), 7.0]]]])
    v = np.array([[[[4.0, 8.0], [0.0, -4.0]]]])
    o = oracle_cross_attention_f64(q, k, v, scale=1.0)
    np.testing.assert_allclose(o.reshape(-1), [1.0, -1.0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("Hq,Hkv", [(24, 8), (4, 4), (6, 1)])
def test_matches_torch_sdpa_with_gqa_and_lengths(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    B, L, d = 3, 37, 16
    q, k, v = _rand(rng, B, Hq, Hkv, L, d)
    lens = np.array([37, 1, 20])
    scale = 0.3
    o = oracle_cross_attention_f64(q, k, v, lens, scale=scale)
    tq = torch.from_numpy(q).unsqueeze(2)                     # [B, Hq, 1, d]
    tk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, 1)  # [B, Hq, L, d]
    tv = torch.from_numpy(v).repeat_interleave(Hq // Hkv, 1)
    mask = torch.arange(L)[None, None, None, :] < torch.from_numpy(lens)[:, None, None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                           scale=scale).squeeze(2).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_equal_scores_average_the_values():
    rng = np.random.default_rng(1)
    q, _, v = _rand(rng, 2, 6, 2, 50, 8)
    k = np.zeros((2, 2, 50, 8))
    o = oracle_cross_attention_f64(q, k, v, np.array([50, 17]))
    np.testing.assert_allclose(o[0], np.repeat(v[0].mean(axis=1), 3, axis=0), atol=1e-14)
    np.testing.assert_allclose(o[1], np.repeat(v[1, :, :17].mean(axis=1), 3, axis=0), atol=1e-14)


def test_single_position_returns_its_value():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 1, 4, 2, 9, 8)
    o = oracle_cross_attention_f64(q, k, v, np.array([1]))
    np.testing.assert_allclose(o[0], np.repeat(v[0, :, 0], 2, axis=0), rtol=0, atol=0)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 2, 1, 40, 16)
    k[0, 0, 23] = 60.0 * q[0, 0] / np.linalg.norm(q[0, 0])  # head 0 score >> the rest
    o = oracle_cross_attention_f64(q, k, v, scale=1.0)
    np.testing.assert_allclose(o[0, 0], v[0, 0, 23], atol=1e-9)


def test_position_permutation_invariance_and_ignored_tail():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 2, 8, 4, 30, 8)
    lens = np.array([30, 12])
    o = oracle_cross_attention_f64(q, k, v, lens)
    perm = rng.permutation(30)
    kp, vp = k.copy(), v.copy()
    kp[0], vp[0] = k[0][:, perm], v[0][:, perm]
    p1 = rng.permutation(12)
    kp[1, :, :12], vp[1, :, :12] = k[1][:, p1], v[1][:, p1]
    kp[1, :, 12:] = 1e6  # beyond the length: never read
    vp[1, :, 12:] = np.nan
    np.testing.assert_allclose(oracle_cross_attention_f64(q, kp, vp, lens), o, rtol=1e-12,
                               atol=1e-13)


def test_heads_of_a_group_share_the_cache():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 1, 24, 8, 16, 8)
    q[0, 4] = q[0, 3]  # heads 3 and 4 share KV head 1
    q[0, 6] = q[0, 3]  # head 6 uses KV head 2
    o = oracle_cross_attention_f64(q, k, v)
    np.testing.assert_array_equal(o[0, 4], o[0, 3])
    assert np.max(np.abs(o[0, 6] - o[0, 3])) > 1e-3


def test_bf16_inputs_widened_exactly():
    from workloads import f32_to_bf16_bits

    rng = np.random.default_rng(6)
    q, k, v = (x.astype(np.float32) for x in _rand(rng, 1, 3, 1, 10, 8))
    qb, kb, vb = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    w = [(x.astype(np.uint32) << 16).view(np.float32).astype(np.float64) for x in (qb, kb, vb)]
    np.testing.assert_array_equal(oracle_cross_attention_f64(qb, kb, vb),
                                  oracle_cross_attention_f64(*w))
