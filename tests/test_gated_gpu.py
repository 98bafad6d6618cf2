"""GPU parity of the gated entry points (retention + output epilogue) against the
fp64 oracle chain: oracle recurrence, then the oracle epilogue (per-head
GroupNorm over dv, optional per-channel affine, swish(gate)).

Bar: eps = max|y - ref| / max|ref| <= 1e-2 for bf16 and <= 1e-4 for fp32, and
the final state as for the plain entry points. Inputs come from seeded
generators, never from the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import oracle_output_gate_f64
from tests.gpu_util import eps, to_dev, to_host
from workloads import f32_to_bf16_bits, make_decode_inputs, make_prefill_inputs, slow_decay_log_gamma

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2
TOL_F32 = 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gret():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import yoco_gated_retention_amd as g

    g.load_library()
    oracle.build_oracle(force=False)
    return g


def seeded_inputs(B, H, N, dk, dv, dtype, seed, s0=True):
    rng = np.random.default_rng(seed)

    def st(x):
        return f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)

    q = st(rng.standard_normal((B, H, N, dk)).astype(np.float32) / np.sqrt(dk))
    k = st(rng.standard_normal((B, H, N, dk)).astype(np.float32) / np.sqrt(dk))
    v = st(rng.standard_normal((B, H, N, dv)).astype(np.float32))
    u = rng.standard_normal((B, H, N))
    lg = (-np.logaddexp(0.0, -u) / 16.0).astype(np.float32)
    S0 = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32) if s0 else None
    gate = st((2.0 * rng.standard_normal((B, H, N, dv))).astype(np.float32))
    w = (1.0 + 0.2 * rng.standard_normal((H, dv))).astype(np.float32)
    b = (0.2 * rng.standard_normal((H, dv))).astype(np.float32)
    return dict(q=q, k=k, v=v, log_gamma=lg), S0, gate, w, b


def check_prefill_gated(gret, d, S0, gate, w, b, norm_eps, chunk, tol, label=""):
    B, H, N, dk = d["q"].shape
    dv = d["v"].shape[3]
    say("prefill_gated %s B=%d H=%d N=%d dk=%d dv=%d chunk=%d affine=%s eps=%g" % (
        label, B, H, N, dk, dv, chunk, w is not None, norm_eps))
    out, st = gret.gret_prefill_gated(
        to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"]), to_dev(d["log_gamma"]), to_dev(gate),
        state_in=None if S0 is None else to_dev(S0),
        norm_weight=None if w is None else to_dev(w), norm_bias=None if b is None else to_dev(b),
        norm_eps=norm_eps, chunk=chunk)
    torch.cuda.synchronize()
    o_ref, s_ref, _ = oracle.oracle_prefill_f64(d["q"], d["k"], d["v"], d["log_gamma"], S0)
    y_ref = oracle_output_gate_f64(o_ref, gate, w, b, eps=norm_eps)
    e_y, e_s = eps(to_host(out), y_ref), eps(to_host(st), s_ref)
    say("   eps_y=%.3e eps_state=%.3e" % (e_y, e_s))
    assert e_y <= tol and e_s <= tol, (e_y, e_s)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("chunk", [64, 256])
def test_prefill_gated_bf16_dims(gret, dk, dv, chunk):
    d, S0, gate, w, b = seeded_inputs(2, 3, 1000, dk, dv, "bf16", seed=dk * 7 + dv + chunk)
    check_prefill_gated(gret, d, S0, gate, w, b, 1e-5, chunk, TOL_BF16, "dims")


@pytest.mark.parametrize("affine", [False, True])
@pytest.mark.parametrize("norm_eps", [1e-5, 0.5])
def test_prefill_gated_bf16_affine_eps(gret, affine, norm_eps):
    d, S0, gate, w, b = seeded_inputs(1, 4, 777, 128, 128, "bf16", seed=11, s0=False)
    check_prefill_gated(gret, d, S0, gate, w if affine else None, b if affine else None,
                        norm_eps, 64, TOL_BF16, "affine")


@pytest.mark.parametrize("chunk", [64, 128])
def test_prefill_gated_f32(gret, chunk):
    d, S0, gate, w, b = seeded_inputs(1, 2, 600, 64, 64, "f32", seed=21 + chunk)
    check_prefill_gated(gret, d, S0, gate, w, b, 1e-5, chunk, TOL_F32, "f32")


def _random_cases(n, seed):
    """Seeded random shapes for the gated prefill: dtype, batch, heads, ragged
    N, dims, chunk, with or without the affine and the initial state, and
    GroupNorm eps from tiny to large."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        cases.append((dtype, int(rng.integers(1, 4)), int(rng.integers(1, 7)),
                      int(rng.integers(1, 2000)), int(rng.choice([64, 128])),
                      int(rng.choice([64, 128])), int(rng.choice([64, 128, 256])),
                      bool(rng.integers(0, 2)), bool(rng.integers(0, 2)),
                      float(rng.choice([1e-6, 1e-5, 1e-2, 0.5])), 13000 + i))
    return cases


@pytest.mark.parametrize("case", _random_cases(10, 20261207),
                         ids=lambda c: "%s_B%dH%dN%d_dk%d_dv%d_c%d" % c[:7])
def test_prefill_gated_random_shapes(gret, case):
    dtype, B, H, N, dk, dv, chunk, affine, s0, norm_eps, seed = case
    d, S0, gate, w, b = seeded_inputs(B, H, N, dk, dv, dtype, seed=seed, s0=s0)
    check_prefill_gated(gret, d, S0, gate, w if affine else None, b if affine else None,
                        norm_eps, chunk, TOL_F32 if dtype == "f32" else TOL_BF16, "random")


def test_prefill_gated_short_rows(gret):
    for N in (1, 63, 65):
        d, S0, gate, w, b = seeded_inputs(1, 3, N, 128, 128, "bf16", seed=N)
        check_prefill_gated(gret, d, S0, gate, w, b, 1e-5, 64, TOL_BF16, "short")


def test_prefill_gated_32k_all_heads(gret):
    d = make_prefill_inputs("prefill_32k")
    rng = np.random.default_rng(2002)
    H, N, dv = d["q"].shape[1], d["q"].shape[2], d["v"].shape[3]
    gate = f32_to_bf16_bits((2.0 * rng.standard_normal((1, H, N, dv))).astype(np.float32))
    w = (1.0 + 0.2 * rng.standard_normal((H, dv))).astype(np.float32)
    b = (0.2 * rng.standard_normal((H, dv))).astype(np.float32)
    check_prefill_gated(gret, d, None, gate, w, b, 1e-5, 64, TOL_BF16, "32k")


def test_prefill_gated_32k_gates_near_one_with_state(gret):
    """The 32K workload (24 heads) with gates near 1 (u ~ N(4, 1), mean
    log-gate about -0.0018) and a nonzero initial state, all heads against
    the oracle chain. A segment of 48 chunks never decays below the survival
    threshold here, so every non-first segment's outputs come from the gated
    prefix launch, from its incoming state."""
    d = make_prefill_inputs("prefill_32k")
    B, H, N, dk = d["q"].shape
    dv = d["v"].shape[3]
    d["log_gamma"] = slow_decay_log_gamma(B, H, N)
    rng = np.random.default_rng(4004)
    S0 = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    gate = f32_to_bf16_bits(rng.standard_normal((B, H, N, dv), dtype=np.float32) * np.float32(2.0))
    w = (1.0 + 0.2 * rng.standard_normal((H, dv))).astype(np.float32)
    b = (0.2 * rng.standard_normal((H, dv))).astype(np.float32)
    check_prefill_gated(gret, d, S0, gate, w, b, 1e-5, 64, TOL_BF16, "32k gates near 1")


@pytest.mark.timeout(900)
def test_prefill_gated_512k_all_heads(gret):
    """The 512K workload through the gated prefill (all 24 heads, the launch
    configuration the benchmark times), every head against the oracle chain,
    eight heads per oracle call. Every head spans about eleven segments, so the
    output-free leading chunks and their recomputation from the incoming state
    are covered."""
    d = make_prefill_inputs("prefill_512k")
    B, H, N, dv = d["q"].shape[0], d["q"].shape[1], d["q"].shape[2], d["v"].shape[3]
    rng = np.random.default_rng(3003)
    gate = f32_to_bf16_bits(rng.standard_normal((B, H, N, dv), dtype=np.float32) * np.float32(2.0))
    w = (1.0 + 0.2 * rng.standard_normal((H, dv))).astype(np.float32)
    b = (0.2 * rng.standard_normal((H, dv))).astype(np.float32)
    say("prefill_gated 512K, all heads on the GPU")
    out, st = gret.gret_prefill_gated(
        to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"]), to_dev(d["log_gamma"]), to_dev(gate),
        norm_weight=to_dev(w), norm_bias=to_dev(b), norm_eps=1e-5, chunk=64)
    torch.cuda.synchronize()
    y, st = to_host(out), to_host(st)
    del out
    worst_y = worst_s = 0.0
    for h0 in range(0, H, 8):
        hs = slice(h0, min(H, h0 + 8))
        sl = lambda a: np.ascontiguousarray(a[:, hs])
        o_ref, s_ref, _ = oracle.oracle_prefill_f64(sl(d["q"]), sl(d["k"]), sl(d["v"]),
                                                    sl(d["log_gamma"]), None)
        y_ref = oracle_output_gate_f64(o_ref, sl(gate), w[hs], b[hs], eps=1e-5)
        del o_ref
        for j in range(y_ref.shape[1]):
            e_y = eps(y[:, h0 + j:h0 + j + 1], y_ref[:, j:j + 1])
            e_s = eps(st[:, h0 + j:h0 + j + 1], s_ref[:, j:j + 1])
            worst_y, worst_s = max(worst_y, e_y), max(worst_s, e_s)
            assert e_y <= TOL_BF16 and e_s <= TOL_BF16, (h0 + j, e_y, e_s)
        say("   heads %d-%d: worst so far eps_y=%.3e eps_state=%.3e" % (
            hs.start, hs.stop - 1, worst_y, worst_s))
        del y_ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_decode_gated_small(gret, dtype, dk, dv):
    rng = np.random.default_rng(dk + 3 * dv + (dtype == "bf16"))
    B, H, steps = 3, 5, 8
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32

    def st(x):
        return f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)

    S = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    w = (1.0 + 0.2 * rng.standard_normal((H, dv))).astype(np.float32)
    b = (0.2 * rng.standard_normal((H, dv))).astype(np.float32)
    state = to_dev(S)
    s64 = S.astype(np.float64)
    for t in range(steps):
        q = st(rng.standard_normal((B, H, dk)).astype(np.float32) / np.sqrt(dk))
        k = st(rng.standard_normal((B, H, dk)).astype(np.float32) / np.sqrt(dk))
        v = st(rng.standard_normal((B, H, dv)).astype(np.float32))
        lg = (-np.logaddexp(0.0, -rng.standard_normal((B, H))) / 16.0).astype(np.float32)
        gate = st((2.0 * rng.standard_normal((B, H, dv))).astype(np.float32))
        affine = t % 2 == 0
        y = gret.gret_decode_step_gated(to_dev(q), to_dev(k), to_dev(v), to_dev(lg), state,
                                        to_dev(gate), norm_weight=to_dev(w) if affine else None,
                                        norm_bias=to_dev(b) if affine else None, norm_eps=1e-5)
        torch.cuda.synchronize()
        o_ref = oracle.oracle_decode_f64(q, k, v, lg, s64)
        y_ref = oracle_output_gate_f64(o_ref, gate, w if affine else None,
                                       b if affine else None, eps=1e-5)
        e = eps(to_host(y), y_ref)
        assert e <= tol, (t, e)
    assert eps(to_host(state), s64) <= tol


@pytest.mark.timeout(900)
def test_decode_gated_b256_1000_steps_all_heads(gret):
    """The decode workload (256 sequences x 24 heads, 1000 steps) through the
    gated step, every sequence, head and step against the oracle chain; the
    gate of each step is a fresh seeded draw."""
    d = make_decode_inputs("decode_b256")
    B, H, dv, steps = d["B"], d["H"], d["dv"], d["steps"]
    rng = np.random.default_rng(5005)
    w = (1.0 + 0.2 * rng.standard_normal((H, dv))).astype(np.float32)
    b = (0.2 * rng.standard_normal((H, dv))).astype(np.float32)
    wd, bd = to_dev(w), to_dev(b)
    state = to_dev(d["state"])
    s64 = d["state"].astype(np.float64)
    y = torch.empty((B, H, dv), dtype=torch.bfloat16, device="cuda")
    worst, worst_t = 0.0, -1
    for t in range(steps):
        gate = f32_to_bf16_bits(rng.standard_normal((B, H, dv), dtype=np.float32) * np.float32(2.0))
        gret.gret_decode_step_gated(to_dev(d["q"][t]), to_dev(d["k"][t]), to_dev(d["v"][t]),
                                    to_dev(d["log_gamma"][t]), state, to_dev(gate),
                                    norm_weight=wd, norm_bias=bd, out=y)
        yh = to_host(y)
        o_ref = oracle.oracle_decode_f64(d["q"][t], d["k"][t], d["v"][t], d["log_gamma"][t], s64)
        e = eps(yh, oracle_output_gate_f64(o_ref, gate, w, b))
        if e > worst:
            worst, worst_t = e, t
    e_s = eps(to_host(state), s64)
    say("decode_gated 256x24x1000, all heads: worst eps_y=%.3e (step %d), state eps=%.3e" % (
        worst, worst_t, e_s))
    assert worst <= TOL_BF16 and e_s <= TOL_BF16
