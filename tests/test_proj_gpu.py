"""GPU parity of gret_head_projection (key projection times key_scale, and the
log-gate log(sigmoid(x W_gamma)) / tau) against the fp64 oracle.

Bar: eps = max|x - ref| / max|ref| <= 1e-2 for the bf16 keys and <= 1e-4 for
the fp32 log-gates (bf16 products accumulated in fp32). Inputs come from
seeded generators, never from the GPU. Shapes span several token and channel
tiles with ragged tails, sequences that straddle a 256-token tile, the gate
tile alone and gate heads beyond one wavefront's 64 channels; the full-size
case (N = 524288, D = 3072, 24 heads of 128) is checked on sampled tokens,
each of which the projection computes independently of the others.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle_head_projection_f64
from tests.gpu_util import eps, to_dev, to_host
from workloads import make_projection_inputs

pytestmark = pytest.mark.gpu

TOL_K = 1e-2
TOL_L = 1e-4


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


def check(gret, B, N, D, H, dk, gate=True, scale=None, tau=16.0, seed=0):
    scale = dk ** -0.5 if scale is None else scale
    say("head_projection B=%d N=%d D=%d H=%d dk=%d gate=%s scale=%g tau=%g seed=%d" % (
        B, N, D, H, dk, gate, scale, tau, seed))
    x, wk, wg = make_projection_inputs(seed, B, N, D, H, dk, gate)
    k, lg = gret.gret_head_projection(to_dev(x), to_dev(wk), None if wg is None else to_dev(wg),
                                      key_scale=scale, temperature=tau, H=H)
    torch.cuda.synchronize()
    k_ref, lg_ref = oracle_head_projection_f64(x, wk, wg, key_scale=scale, temperature=tau, H=H)
    e_k = eps(to_host(k), k_ref)
    e_l = eps(to_host(lg), lg_ref) if gate else 0.0
    say("   eps_k=%.3e eps_log_gamma=%.3e" % (e_k, e_l))
    assert e_k <= TOL_K and e_l <= TOL_L, (e_k, e_l)
    if not gate:
        assert lg is None


@pytest.mark.parametrize("B,N,D,H,dk", [
    (1, 256, 128, 2, 128),     # one token tile, one channel tile, one pipeline round
    (1, 1000, 384, 3, 128),    # ragged token tail, 384 channels = 1.5 channel tiles
    (2, 300, 256, 4, 64),      # sequences straddle a token tile
    (3, 77, 512, 5, 32),       # short sequences, dk 32, 160 channels
    (1, 700, 1024, 24, 128),   # the retention's head layout at a small hidden size
])
def test_projection_with_gate(gret, B, N, D, H, dk):
    check(gret, B, N, D, H, dk, seed=B * 1000 + N + D + H + dk)


def _random_cases(n, seed):
    """Seeded random shapes: batch, ragged sequences, hidden sizes that are
    multiples of 128, dk multiples of 16 up to 256, gate heads up to 64, with
    and without the gate, and other scales and temperatures."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        cases.append((int(rng.integers(1, 4)), int(rng.integers(1, 1200)),
                      128 * int(rng.integers(1, 9)), int(rng.integers(1, 65)),
                      16 * int(rng.integers(1, 17)), bool(rng.random() < 0.75),
                      float(rng.uniform(0.05, 1.0)), float(rng.choice([1.0, 4.0, 16.0])),
                      11000 + i))
    return cases


@pytest.mark.parametrize("case", _random_cases(12, 20261206),
                         ids=lambda c: "B%dN%dD%dH%d_dk%d_gate%d" % c[:6])
def test_projection_random_shapes(gret, case):
    B, N, D, H, dk, gate, scale, tau, seed = case
    check(gret, B, N, D, H, dk, gate=gate, scale=scale, tau=tau, seed=seed)


def test_projection_gate_heads_beyond_one_wavefront(gret):
    # 100 gate heads: channels 64..99 of the gate tile fall to a second wavefront
    check(gret, 1, 520, 256, 100, 16, seed=77)


def test_projection_without_gate(gret):
    check(gret, 2, 513, 640, 6, 128, gate=False, scale=1.0, seed=5)


@pytest.mark.parametrize("tau", [1.0, 16.0])
def test_projection_temperature(gret, tau):
    check(gret, 1, 300, 256, 8, 64, tau=tau, scale=0.5, seed=int(tau))


def test_projection_single_token(gret):
    check(gret, 1, 1, 128, 1, 16, seed=3)


def test_projection_large_logits(gret):
    # gate logits of magnitude ~40: log-sigmoid near 0 and near u / tau
    x, wk, wg = make_projection_inputs(9, 1, 400, 256, 8, 64)
    wg40 = (wg.astype(np.uint32) << 16).view(np.float32) * np.float32(40.0)
    from workloads import f32_to_bf16_bits

    wg40 = f32_to_bf16_bits(wg40)
    k, lg = gret.gret_head_projection(to_dev(x), to_dev(wk), to_dev(wg40), key_scale=0.125,
                                      temperature=16.0)
    torch.cuda.synchronize()
    k_ref, lg_ref = oracle_head_projection_f64(x, wk, wg40, key_scale=0.125, temperature=16.0)
    e_k, e_l = eps(to_host(k), k_ref), eps(to_host(lg), lg_ref)
    say("large logits: eps_k=%.3e eps_log_gamma=%.3e max|u|=%.1f" % (
        e_k, e_l, 16 * float(np.abs(lg_ref).max())))
    assert np.isfinite(to_host(lg)).all()
    assert e_k <= TOL_K and e_l <= TOL_L


def test_projection_full_size_sampled(gret):
    """The benchmark's shape (B=1, N=524288, D=3072, 24 heads of 128, gate),
    inputs drawn on the device by a seeded generator; the oracle recomputes
    16384 sampled tokens (the first and last tiles' edges included)."""
    B, N, D, H, dk = 1, 524288, 3072, 24, 128
    say("head_projection full size B=%d N=%d D=%d H=%d dk=%d" % (B, N, D, H, dk))
    g = torch.Generator(device="cuda").manual_seed(6006)
    x = torch.randn((B, N, D), generator=g, device="cuda").to(torch.bfloat16)
    wk = (torch.randn((H * dk, D), generator=g, device="cuda") * D ** -0.5).to(torch.bfloat16)
    wg = (torch.randn((H, D), generator=g, device="cuda") * D ** -0.5).to(torch.bfloat16)
    k, lg = gret.gret_head_projection(x, wk, wg, key_scale=dk ** -0.5, temperature=16.0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    idx = np.unique(np.concatenate([np.arange(0, 8), np.arange(N - 8, N), [255, 256, 257],
                                    rng.integers(0, N, 16384 - 19)]))
    ti = torch.from_numpy(idx).cuda()
    xs = to_host(x[0, ti].contiguous())[None]
    k_ref, lg_ref = oracle_head_projection_f64(xs, to_host(wk), to_host(wg),
                                               key_scale=dk ** -0.5, temperature=16.0)
    ks = to_host(k[0][:, ti].contiguous())[None]
    ls = to_host(lg[0][:, ti].contiguous())[None]
    e_k, e_l = eps(ks, k_ref), eps(ls, lg_ref)
    say("   sampled %d tokens: eps_k=%.3e eps_log_gamma=%.3e" % (len(idx), e_k, e_l))
    assert e_k <= TOL_K and e_l <= TOL_L
    del x, k, lg
    torch.cuda.empty_cache()


def test_projection_feeds_retention(gret):
    """The projection's outputs are the retention's key and log-gate inputs:
    project keys and log-gates on the GPU, run the chunkwise prefill on them,
    and compare with the oracle projection followed by the oracle recurrence
    (queries and values drawn directly, as the projection of x by other
    weights would give)."""
    import oracle
    from workloads import f32_to_bf16_bits

    B, N, D, H, dk = 1, 700, 512, 4, 128
    x, wk, wg = make_projection_inputs(31, B, N, D, H, dk)
    rng = np.random.default_rng(32)
    q = f32_to_bf16_bits((rng.standard_normal((B, H, N, dk)) / np.sqrt(dk)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((B, H, N, dk)).astype(np.float32))
    k_dev, lg_dev = gret.gret_head_projection(to_dev(x), to_dev(wk), to_dev(wg),
                                              key_scale=dk ** -0.5, temperature=16.0)
    out, st = gret.gret_prefill(to_dev(q), k_dev, to_dev(v), lg_dev, None, chunk=64)
    torch.cuda.synchronize()
    oracle.build_oracle(force=False)
    k_ref, lg_ref = oracle_head_projection_f64(x, wk, wg, key_scale=dk ** -0.5, temperature=16.0)
    # the retention oracle takes the stored types: keys in bf16, log-gates in fp32
    k_bits = f32_to_bf16_bits(k_ref.astype(np.float32))
    o_ref, s_ref, _ = oracle.oracle_prefill_f64(q, k_bits, v, lg_ref.astype(np.float32))
    e_o, e_s = eps(to_host(out), o_ref), eps(to_host(st), s_ref)
    say("projection -> prefill: eps_out=%.3e eps_state=%.3e" % (e_o, e_s))
    assert e_o <= TOL_K and e_s <= TOL_K
