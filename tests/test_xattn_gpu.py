"""GPU parity of the Cross-Decoder decode attention (gret_cross_attention_decode)
against the fp64 oracle on seeded inputs: eps = max|out - ref| / max|ref| <=
1e-2 (bf16 operands, bf16 probabilities, fp32 softmax and sums)."""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle_cross_attention_f64
from tests.gpu_util import eps, to_dev, to_host
from workloads import f32_to_bf16_bits

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


def inputs(B, Hq, Hkv, L, d, seed):
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, d)).astype(np.float32))
    k = f32_to_bf16_bits(rng.standard_normal((B, Hkv, L, d)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((B, Hkv, L, d)).astype(np.float32))
    return q, k, v


def check(gret, B, Hq, Hkv, L, d, lengths=None, scale=None, seed=0, label=""):
    q, k, v = inputs(B, Hq, Hkv, L, d, seed)
    lens_dev = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device="cuda")
    say("xattn %s B=%d Hq=%d Hkv=%d L=%d d=%d lengths=%s" % (label, B, Hq, Hkv, L, d,
                                                            None if lengths is None else
                                                            list(lengths)[:4]))
    out = gret.gret_cross_attention_decode(to_dev(q), to_dev(k), to_dev(v), lens_dev, scale)
    torch.cuda.synchronize()
    ref = oracle_cross_attention_f64(q, k, v, lengths, scale)
    e = eps(to_host(out), ref)
    say("   eps=%.3e" % e)
    assert e <= TOL, e
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(24, 8), (4, 4), (16, 1)])
def test_shapes(gret, d, Hq, Hkv):
    check(gret, 2, Hq, Hkv, 3001, d, seed=d + Hq, label="shapes")


@pytest.mark.parametrize("L", [1, 2, 31, 32, 33, 127, 129, 513])
def test_short_caches(gret, L):
    check(gret, 1, 24, 8, L, 128, seed=L, label="short")


def test_per_sequence_lengths(gret):
    check(gret, 4, 24, 8, 3000, 128, lengths=[3000, 1, 1777, 129], seed=7, label="lengths")


def test_scale_argument(gret):
    check(gret, 2, 6, 2, 900, 64, scale=0.02, seed=8, label="scale")
    check(gret, 2, 6, 2, 900, 64, scale=0.4, seed=9, label="scale")


def _random_cases(n, seed):
    """Seeded random shapes: group sizes up to the supported 16, batches with
    per-sequence lengths from 1 to L, short and long caches, both d, and an
    explicit scale on some."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B, Hkv = int(rng.integers(1, 5)), int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
        L = int(rng.integers(1, 6000))
        lengths = None
        if rng.random() < 0.5:
            lengths = [int(x) for x in rng.integers(1, L + 1, B)]
        scale = float(rng.uniform(0.02, 0.3)) if rng.random() < 0.3 else None
        cases.append((B, Hkv * G, Hkv, L, int(rng.choice([64, 128])), lengths, scale, 9000 + i))
    return cases


@pytest.mark.parametrize("case", _random_cases(12, 20261204),
                         ids=lambda c: "B%dHq%dHkv%dL%d_d%d" % c[:5])
def test_random_shapes(gret, case):
    B, Hq, Hkv, L, d, lengths, scale, seed = case
    check(gret, B, Hq, Hkv, L, d, lengths=lengths, scale=scale, seed=seed, label="random")


def test_deterministic(gret):
    q, k, v = inputs(1, 24, 8, 2048, 128, 10)
    a = gret.gret_cross_attention_decode(to_dev(q), to_dev(k), to_dev(v))
    b = gret.gret_cross_attention_decode(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_512k_context_all_heads(gret):
    # the benchmarked shape: one sequence, 24 query / 8 KV heads, 524288 cached positions
    check(gret, 1, 24, 8, 524288, 128, seed=11, label="512k")


def test_batch_of_32k_contexts(gret):
    check(gret, 16, 24, 8, 32768, 128, lengths=[32768 - 97 * i for i in range(16)], seed=12,
          label="16x32k")


@pytest.mark.timeout(900)
def test_cache_longer_than_2_pow_23(gret):
    """One sequence whose cache holds 2^23 + 2^20 + 33 positions (past any
    32-bit byte offset of the cache's rows; every range addresses its
    positions from its own first one), 8 query heads on one KV head, inputs
    drawn on the device by a seeded generator; all positions, then a
    shorter valid length."""
    B, Hq, Hkv, L, d = 1, 8, 1, (1 << 23) + (1 << 20) + 33, 128
    say("xattn long cache B=%d Hq=%d Hkv=%d L=%d d=%d" % (B, Hq, Hkv, L, d))
    g = torch.Generator(device="cuda").manual_seed(2525)
    q = torch.randn((B, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16)
    hq, hk, hv = to_host(q), to_host(k), to_host(v)
    for lengths in (None, [L - 12345]):
        lens_dev = None if lengths is None else torch.tensor(lengths, dtype=torch.int32,
                                                             device="cuda")
        out = gret.gret_cross_attention_decode(q, k, v, lens_dev, None)
        torch.cuda.synchronize()
        e = eps(to_host(out), oracle_cross_attention_f64(hq, hk, hv, lengths, None))
        say("   lengths=%s eps=%.3e" % (lengths, e))
        assert e <= TOL, e
    del q, k, v
    torch.cuda.empty_cache()
