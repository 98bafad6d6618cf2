"""GPU parity of the sliding-window-attention entry points (prefill, the ring
it leaves, decode steps over the ring) against the fp64 oracle.

Bar: eps = max|x - ref| / max|ref| <= 1e-2 (bf16 inputs and outputs, fp32
softmax and accumulation); the ring contents are copies and must match
bit for bit. Inputs come from seeded generators, never from the GPU. Shapes
cover ragged query tiles, windows below, equal to and above the 256-query
tile and the prompt, d = 64 and 128, grouped query heads, sequences decoding
at different positions (ring partly filled and wrapped), and the full-size
prompt (524288 positions, 24 heads, window 1024) on sampled rows of every head, each of
which depends only on its own window.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle_swa_decode_f64, oracle_swa_prefill_f64, oracle_swa_ring_f64
from tests.gpu_util import eps, to_dev, to_host
from workloads import bf16_bits_to_f32, make_attention_inputs

pytestmark = pytest.mark.gpu

TOL = 1e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gret():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import yoco_gated_retention_amd as g

    g.load_library()
    return g


@pytest.mark.parametrize("B,Hq,Hkv,N,d,W", [
    (1, 2, 2, 300, 128, 64),
    (2, 4, 2, 1000, 128, 256),
    (1, 3, 1, 700, 64, 100),
    (1, 2, 2, 2000, 128, 1024),
    (1, 1, 1, 50, 128, 1),
    (1, 2, 2, 130, 128, 4096),
    (1, 2, 1, 1, 64, 16),
    (1, 2, 2, 777, 64, 1024),
])
def test_swa_prefill_and_ring(gret, B, Hq, Hkv, N, d, W):
    say("swa_prefill B=%d Hq=%d Hkv=%d N=%d d=%d window=%d" % (B, Hq, Hkv, N, d, W))
    q, k, v = make_attention_inputs(N + W + d, B, Hq, Hkv, N, d)
    rk = torch.zeros((B, Hkv, W, d), dtype=torch.bfloat16, device="cuda")
    rv = torch.zeros_like(rk)
    out = gret.gret_swa_prefill(to_dev(q), to_dev(k), to_dev(v), W, k_ring=rk, v_ring=rv)
    torch.cuda.synchronize()
    ref = oracle_swa_prefill_f64(q, k, v, W)
    e = eps(to_host(out), ref)
    say("   eps_out=%.3e" % e)
    assert e <= TOL
    wk, wv = oracle_swa_ring_f64(k, v, W)
    np.testing.assert_array_equal(bf16_bits_to_f32(to_host(rk)), wk)
    np.testing.assert_array_equal(bf16_bits_to_f32(to_host(rv)), wv)


def _random_cases(n, seed):
    """Seeded random shapes: batch, grouped heads, ragged prompts and windows
    from 1 to beyond the prompt, both d."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        Hkv = int(rng.integers(1, 4))
        N = int(rng.integers(1, 2500))
        W = int(rng.integers(1, 3000))
        cases.append((int(rng.integers(1, 3)), Hkv * int(rng.integers(1, 4)), Hkv, N,
                      int(rng.choice([64, 128])), W))
    return cases


@pytest.mark.parametrize("B,Hq,Hkv,N,d,W", _random_cases(10, 20261205))
def test_swa_prefill_and_ring_random(gret, B, Hq, Hkv, N, d, W):
    test_swa_prefill_and_ring(gret, B, Hq, Hkv, N, d, W)


def test_swa_prefill_without_rings(gret):
    q, k, v = make_attention_inputs(3, 1, 2, 2, 600, 128)
    out = gret.gret_swa_prefill(to_dev(q), to_dev(k), to_dev(v), 300)
    torch.cuda.synchronize()
    assert eps(to_host(out), oracle_swa_prefill_f64(q, k, v, 300)) <= TOL


@pytest.mark.parametrize("d,W,Hq,Hkv", [(128, 64, 4, 2), (64, 32, 2, 2), (128, 1024, 3, 1)])
def test_swa_decode_steps(gret, d, W, Hq, Hkv):
    """Prefill each sequence to its own length, then decode 6 steps; sequence
    prompts below, at and above the window."""
    lens = [W // 2, W, W + 37]
    B, steps = len(lens), 6
    T = max(lens) + steps
    say("swa_decode d=%d window=%d Hq=%d Hkv=%d prompts=%s" % (d, W, Hq, Hkv, lens))
    q, k, v = make_attention_inputs(d + W + Hq, B, Hq, Hkv, T, d)
    rk = torch.zeros((B, Hkv, W, d), dtype=torch.bfloat16, device="cuda")
    rv = torch.zeros_like(rk)
    for b, n in enumerate(lens):
        gret.gret_swa_prefill(to_dev(q[b:b + 1, :, :n]), to_dev(k[b:b + 1, :, :n]),
                              to_dev(v[b:b + 1, :, :n]), W, k_ring=rk[b:b + 1], v_ring=rv[b:b + 1])
    ref = oracle_swa_prefill_f64(q, k, v, W)  # row t of sequence b is its step at position t
    ring_k = np.zeros((B, Hkv, W, d))
    ring_v = np.zeros((B, Hkv, W, d))
    for b, n in enumerate(lens):
        a, c = oracle_swa_ring_f64(k[b:b + 1, :, :n], v[b:b + 1, :, :n], W)
        ring_k[b], ring_v[b] = a[0], c[0]
    worst = 0.0
    for s in range(steps):
        pos = np.array([n + s for n in lens])
        qs = np.ascontiguousarray(q[np.arange(B), :, pos])
        ks = np.ascontiguousarray(k[np.arange(B), :, pos])
        vs = np.ascontiguousarray(v[np.arange(B), :, pos])
        out = gret.gret_swa_decode_step(to_dev(qs), to_dev(ks), to_dev(vs), rk, rv,
                                        torch.from_numpy(pos.astype(np.int32)).cuda())
        torch.cuda.synchronize()
        o_ref, ring_k, ring_v = oracle_swa_decode_f64(qs, ks, vs, ring_k, ring_v, pos)
        np.testing.assert_allclose(o_ref, ref[np.arange(B), :, pos], rtol=1e-9, atol=1e-12)
        worst = max(worst, eps(to_host(out), o_ref))
    say("   worst eps_out=%.3e" % worst)
    assert worst <= TOL
    np.testing.assert_array_equal(bf16_bits_to_f32(to_host(rk)), ring_k)
    np.testing.assert_array_equal(bf16_bits_to_f32(to_host(rv)), ring_v)


def test_swa_prefill_full_size_sampled(gret):
    """524288 positions, 24 heads of 128, window 1024, inputs drawn on the
    device by a seeded generator; on every head, 512 sampled rows (the window
    and tile edges included) against the oracle over each row's window."""
    B, H, N, d, W = 1, 24, 524288, 128, 1024
    say("swa_prefill full size B=%d H=%d N=%d d=%d window=%d" % (B, H, N, d, W))
    g = torch.Generator(device="cuda").manual_seed(8008)
    q = torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
    out = gret.gret_swa_prefill(q, k, v, W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    edges = [0, 1, 255, 256, 1023, 1024, 1025, N - 1]
    worst = 0.0
    n_rows = 0
    for h in range(H):
        rows = np.unique(np.concatenate([edges, rng.integers(0, N, 512 - len(edges))]))
        ti = torch.from_numpy(rows).cuda()
        qs = to_host(q[0, h, ti].contiguous())[None, None]
        ks = to_host(k[0, h].contiguous())[None, None]
        vs = to_host(v[0, h].contiguous())[None, None]
        ref = oracle_swa_prefill_f64(qs, ks, vs, W, rows=rows)
        got = to_host(out[0, h, ti].contiguous())[None, None]
        worst = max(worst, eps(got, ref))
        n_rows += len(rows)
    say("   sampled %d rows over %d heads: worst eps_out=%.3e" % (n_rows, H, worst))
    assert worst <= TOL
    del q, k, v, out
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_swa_prefill_longer_than_2_pow_23(gret):
    """One head of 2^23 + 2^20 + 77 positions (past any 32-bit byte offset of
    the head's rows), window 1024, with the rings: sampled rows (around 2^23,
    at query-tile edges, the last rows and 200 random ones) against the oracle
    over each row's window, and the rings against the prompt's last 1024
    keys and values (slot p mod 1024 holds position p)."""
    N, d, W = (1 << 23) + (1 << 20) + 77, 128, 1024
    say("swa_prefill one head N=%d d=%d window=%d" % (N, d, W))
    g = torch.Generator(device="cuda").manual_seed(2424)
    q = torch.randn((1, 1, N, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((1, 1, N, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((1, 1, N, d), generator=g, device="cuda").to(torch.bfloat16)
    rk = torch.zeros((1, 1, W, d), dtype=torch.bfloat16, device="cuda")
    rv = torch.zeros_like(rk)
    out = gret.gret_swa_prefill(q, k, v, W, k_ring=rk, v_ring=rv)
    torch.cuda.synchronize()
    rng = np.random.default_rng(24)
    ends = np.unique(np.concatenate([
        [0, 255, 256, W, (1 << 23) - 256, (1 << 23) - 1, 1 << 23, (1 << 23) + 1, N - 2, N - 1],
        rng.integers(0, N, 200)]))
    lo = np.maximum(ends - (W - 1), 0)
    need = np.unique(np.concatenate([np.arange(a, b + 1) for a, b in zip(lo, ends)]))
    ti = torch.from_numpy(need).cuda()
    # a compact prompt holding just the needed rows; row r of it is position need[r]
    hq, hk, hv = (to_host(t[0, 0, ti].contiguous()) for t in (q, k, v))
    worst = 0.0
    for e, a in zip(ends, lo):
        r0, r1 = np.searchsorted(need, [a, e])
        # rows a..e are contiguous in `need`: a prompt of e - a + 1 rows whose
        # last row is position e (its window starts at a)
        qq = np.zeros((1, 1, r1 - r0 + 1, d), np.uint16)
        qq[0, 0, -1] = hq[r1]
        ref = oracle_swa_prefill_f64(qq, hk[None, None, r0:r1 + 1], hv[None, None, r0:r1 + 1], W,
                                     rows=[r1 - r0])[0, 0, 0]
        got = to_host(out[0, 0, int(e)].contiguous())
        worst = max(worst, eps(got, ref))
    say("   %d sampled rows: worst eps_out=%.3e" % (len(ends), worst))
    assert worst <= TOL
    slots = torch.arange(N - W, N, device="cuda") % W
    assert torch.equal(rk[0, 0, slots], k[0, 0, N - W:]) and torch.equal(rv[0, 0, slots], v[0, 0, N - W:])
    del q, k, v, out, rk, rv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("q_scale", [8.0, 30.0])
def test_swa_prefill_peaked_scores(gret, q_scale):
    """Scores with standard deviation 8 and 30: the running softmax maximum
    jumps often and far, so the output rescaling path runs many times (and
    weights far below the maximum underflow to 0)."""
    B, Hq, Hkv, N, d, W = 1, 2, 1, 1500, 128, 512
    q, k, v = make_attention_inputs(int(q_scale), B, Hq, Hkv, N, d)
    from workloads import f32_to_bf16_bits

    q = f32_to_bf16_bits(bf16_bits_to_f32(q) * np.float32(q_scale))
    say("swa_prefill peaked scores q_scale=%g" % q_scale)
    out = gret.gret_swa_prefill(to_dev(q), to_dev(k), to_dev(v), W)
    torch.cuda.synchronize()
    e = eps(to_host(out), oracle_swa_prefill_f64(q, k, v, W))
    say("   eps_out=%.3e" % e)
    assert e <= TOL
