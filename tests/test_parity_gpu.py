"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: eps = max|x - ref| / max|ref| <= 1e-2 for bf16 inputs with fp32
accumulation and <= 1e-4 on the fp32 path, for outputs and final states; the
decode check holds per step. Inputs come from the shared seeded generator,
never from the GPU.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import oracle_output_gate_f64
from tests.gpu_util import as_f64, eps, stats_eps, to_dev, to_host
from workloads import CONFIGS, make_decode_inputs, make_prefill_inputs, slow_decay_log_gamma

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


def gpu_prefill(gret, d, chunk, s0=None, state_out=True):
    q, k, v = to_dev(d["q"]), to_dev(d["k"]), to_dev(d["v"])
    lg = to_dev(d["log_gamma"])
    si = None if s0 is None else to_dev(s0)
    out, st = gret.gret_prefill(q, k, v, lg, si, chunk=chunk)
    torch.cuda.synchronize()
    return to_host(out), to_host(st)


def check_prefill(gret, d, chunk, tol, s0=None, label=""):
    say("prefill %s B=%d H=%d N=%d dk=%d dv=%d chunk=%d" % (
        label, d["q"].shape[0], d["q"].shape[1], d["q"].shape[2], d["q"].shape[3],
        d["v"].shape[3], chunk))
    out, st = gpu_prefill(gret, d, chunk, s0)
    o_ref, s_ref, _ = oracle.oracle_prefill_f64(d["q"], d["k"], d["v"], d["log_gamma"], s0)
    e_o, e_s = eps(out, o_ref), eps(st, s_ref)
    say("   eps_out=%.3e eps_state=%.3e" % (e_o, e_s))
    assert e_o <= tol and e_s <= tol, (e_o, e_s)
    return out, st, o_ref, s_ref


def small_inputs(B, H, N, dk, dv, dtype="bf16", seed=5, s0=True, lg_mode="gate"):
    rng = np.random.default_rng(seed)
    from workloads import f32_to_bf16_bits

    def st(x):
        return f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)

    q = st(rng.standard_normal((B, H, N, dk)).astype(np.float32) / np.sqrt(dk))
    k = st(rng.standard_normal((B, H, N, dk)).astype(np.float32) / np.sqrt(dk))
    v = st(rng.standard_normal((B, H, N, dv)).astype(np.float32))
    if lg_mode == "gate":
        u = rng.standard_normal((B, H, N))
        lg = (-np.logaddexp(0.0, -u) / 16.0).astype(np.float32)
    elif lg_mode == "one":
        lg = np.zeros((B, H, N), np.float32)
    elif lg_mode == "zero":
        lg = np.full((B, H, N), -np.inf, np.float32)
    elif lg_mode == "mixed":
        lg = rng.uniform(-1.0, 0.0, (B, H, N)).astype(np.float32)
        lg[rng.random((B, H, N)) < 0.05] = -np.inf
    S0 = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32) if s0 else None
    return dict(q=q, k=k, v=v, log_gamma=lg), S0


# ---------------------------------------------------------------- fp32 path

def test_tiny_f32_prefill_then_16_decode_steps(gret):
    d = make_prefill_inputs("tiny_f32")
    out, st, o_ref, s_ref = check_prefill(gret, d, 64, TOL_F32, label="tiny_f32")
    state = to_dev(st)
    s64 = s_ref.copy()
    for t in range(CONFIGS["tiny_f32"]["decode_steps"]):
        o = gret.gret_decode_step(to_dev(d["dec_q"][t]), to_dev(d["dec_k"][t]),
                                  to_dev(d["dec_v"][t]), to_dev(d["dec_log_gamma"][t]), state)
        torch.cuda.synchronize()
        o_r = oracle.oracle_decode_f64(d["dec_q"][t], d["dec_k"][t], d["dec_v"][t],
                                       d["dec_log_gamma"][t], s64)
        assert eps(to_host(o), o_r) <= TOL_F32
    assert eps(to_host(state), s64) <= TOL_F32


@pytest.mark.parametrize("dk,dv,chunk", [(64, 128, 128), (128, 64, 256), (128, 128, 64)])
def test_fp32_dims_and_chunks(gret, dk, dv, chunk):
    d, S0 = small_inputs(1, 2, 700, dk, dv, dtype="f32", seed=dk + dv + chunk)
    check_prefill(gret, d, chunk, TOL_F32, S0, label="f32")


@pytest.mark.parametrize("N", [1, 17, 64, 65, 128, 129, 191, 256, 257])
@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_fp32_short_lengths(gret, N, chunk, dk, dv):
    # the fp32 kernel stages 64-position sub-chunks: lengths that end inside,
    # at and just past a sub-chunk or a chunk, with an initial state
    d, S0 = small_inputs(1, 2, N, dk, dv, dtype="f32", seed=7 * N + chunk + dk)
    check_prefill(gret, d, chunk, TOL_F32, S0, label="f32 short")


@pytest.mark.parametrize("lg_mode", ["one", "zero", "mixed"])
@pytest.mark.parametrize("chunk", [64, 256])
def test_fp32_gate_regimes(gret, lg_mode, chunk):
    # gates = 1 (no decay), gates = 0 (a reset at every position) and mixed
    d, S0 = small_inputs(2, 2, 300, 128, 128, dtype="f32", seed=31 + chunk, lg_mode=lg_mode)
    check_prefill(gret, d, chunk, TOL_F32, S0, label="f32 " + lg_mode)


# ---------------------------------------------------------------- bf16 path

@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_bf16_ragged_multi_tile(gret, chunk, dk, dv):
    d, S0 = small_inputs(2, 3, 1000, dk, dv, seed=chunk + dk + 3 * dv)
    check_prefill(gret, d, chunk, TOL_BF16, S0, label="ragged")


@pytest.mark.parametrize("N", [1, 2, 17, 63, 64, 65, 129, 255, 257])
@pytest.mark.parametrize("chunk", [64, 256])
def test_bf16_short_lengths(gret, N, chunk):
    d, S0 = small_inputs(1, 2, N, 128, 128, seed=N)
    check_prefill(gret, d, chunk, TOL_BF16, S0, label="short")


def test_bf16_many_heads_one_chunk_each(gret):
    # every (head, chunk) pair becomes its own workgroup range
    d, S0 = small_inputs(4, 24, 60, 128, 128, seed=9)
    check_prefill(gret, d, 64, TOL_BF16, S0, label="many-heads")


@pytest.mark.parametrize("chunk", [64, 256])
def test_bf16_gate_one_long(gret, chunk):
    # gamma = 1: incoming states never decay, every segment is recomputed
    d, S0 = small_inputs(1, 2, 16384, 128, 128, seed=21, lg_mode="one")
    check_prefill(gret, d, chunk, TOL_BF16, S0, label="gate-one")


def test_bf16_gate_zero_and_mixed_resets(gret):
    d, S0 = small_inputs(1, 2, 3000, 128, 128, seed=22, lg_mode="zero")
    check_prefill(gret, d, 64, TOL_BF16, S0, label="gate-zero")
    d, S0 = small_inputs(1, 4, 5000, 128, 128, seed=23, lg_mode="mixed")
    check_prefill(gret, d, 128, TOL_BF16, S0, label="mixed")


def test_bf16_split_prefill_then_decode(gret):
    d, S0 = small_inputs(1, 4, 3000, 128, 128, seed=31)
    N1 = 1777
    head = {key: val[:, :, :N1] for key, val in d.items()}
    tail = {key: val[:, :, N1:] for key, val in d.items()}
    o1, s1 = gpu_prefill(gret, head, 64, S0)
    o2, s2 = gpu_prefill(gret, tail, 128, s1)
    o_ref, s_ref, _ = oracle.oracle_prefill_f64(d["q"], d["k"], d["v"], d["log_gamma"], S0)
    assert eps(np.concatenate([as_f64(o1), as_f64(o2)], axis=2), o_ref) <= TOL_BF16
    assert eps(s2, s_ref) <= TOL_BF16
    # continue with decode steps from the GPU state
    state = to_dev(s2)
    s64 = s_ref.copy()
    dd, _ = small_inputs(1, 4, 8, 128, 128, seed=32, s0=False)
    for t in range(8):
        args = [np.ascontiguousarray(dd[key][:, :, t]) for key in ("q", "k", "v", "log_gamma")]
        o = gret.gret_decode_step(*(to_dev(a) for a in args), state)
        torch.cuda.synchronize()
        o_r = oracle.oracle_decode_f64(*args, s64)
        assert eps(to_host(o), o_r) <= TOL_BF16
    assert eps(to_host(state), s64) <= TOL_BF16


def _random_cases(n, seed):
    """Seeded random shapes: batch and head counts that split sequences across
    segment ranges, ragged N, every head-dim pair and chunk size, each gate
    regime, with or without an initial state."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        modes = ["gate", "mixed"] if dtype == "f32" else ["gate", "gate", "mixed", "one", "zero"]
        cases.append((dtype, int(rng.integers(1, 4)), int(rng.integers(1, 8)),
                      int(rng.integers(1, 2500)), int(rng.choice([64, 128])),
                      int(rng.choice([64, 128])), int(rng.choice([64, 128, 256])),
                      str(rng.choice(modes)), bool(rng.integers(0, 2)), 7000 + i))
    return cases


@pytest.mark.parametrize("case", _random_cases(16, 20261203),
                         ids=lambda c: "%s_B%dH%dN%d_dk%d_dv%d_c%d_%s_s0%d" % c[:9])
def test_random_shapes_prefill_then_decode(gret, case):
    dtype, B, H, N, dk, dv, chunk, lg_mode, s0, seed = case
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    d, S0 = small_inputs(B, H, N, dk, dv, dtype=dtype, seed=seed, s0=s0, lg_mode=lg_mode)
    _, st, _, s_ref = check_prefill(gret, d, chunk, tol, S0, label="random")
    # three decode steps from the GPU's final state, against the oracle's
    state = to_dev(st)
    s64 = s_ref.copy()
    dd, _ = small_inputs(B, H, 3, dk, dv, dtype=dtype, seed=seed + 500, s0=False, lg_mode=lg_mode)
    for t in range(3):
        args = [np.ascontiguousarray(dd[key][:, :, t]) for key in ("q", "k", "v", "log_gamma")]
        o = gret.gret_decode_step(*(to_dev(a) for a in args), state)
        torch.cuda.synchronize()
        o_r = oracle.oracle_decode_f64(*args, s64)
        assert eps(to_host(o), o_r) <= tol, ("decode step", t)
    assert eps(to_host(state), s64) <= tol


def test_bf16_in_place_state_and_no_state_out(gret):
    d, S0 = small_inputs(2, 2, 900, 128, 128, seed=41)
    q, k, v, lg = (to_dev(d[key]) for key in ("q", "k", "v", "log_gamma"))
    st = to_dev(S0)
    out, st2 = gret.gret_prefill(q, k, v, lg, st, chunk=64, state_out=st)
    torch.cuda.synchronize()
    assert st2.data_ptr() == st.data_ptr()
    o_ref, s_ref, _ = oracle.oracle_prefill_f64(d["q"], d["k"], d["v"], d["log_gamma"], S0)
    assert eps(to_host(out), o_ref) <= TOL_BF16
    assert eps(to_host(st), s_ref) <= TOL_BF16
    # state_out = NULL at the ABI: outputs only
    lib = gret.load_library()
    import ctypes
    out2 = torch.empty_like(out)
    need = gret.gret_prefill_workspace_bytes(2, 2, 900, 128, 128, 64, 1)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st0 = to_dev(S0)
    rc = lib.gret_prefill(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                          ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(lg.data_ptr()),
                          ctypes.c_void_p(st0.data_ptr()), ctypes.c_void_p(out2.data_ptr()),
                          None, 2, 2, 900, 128, 128, 64, 1, ctypes.c_void_p(ws.data_ptr()), need,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(out2, out)


def test_bf16_bitwise_deterministic(gret):
    d, S0 = small_inputs(1, 8, 20000, 128, 128, seed=51)
    a = gpu_prefill(gret, d, 64, S0)
    b = gpu_prefill(gret, d, 64, S0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------- full-size workloads (configs)

@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_prefill_32k_full(gret, chunk):
    d = make_prefill_inputs("prefill_32k")
    say("prefill_32k chunk=%d" % chunk)
    out, st = gpu_prefill(gret, d, chunk)
    _, s_ref, stats = oracle.oracle_prefill_f64(d["q"], d["k"], d["v"], d["log_gamma"],
                                                want_out=False, compare=out)
    e_o, e_s = stats_eps(stats), eps(st, s_ref)
    say("   eps_out=%.3e eps_state=%.3e" % (e_o, e_s))
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16


def _full_check(gret, workload, chunk, first_chunk=False, log_gamma=None):
    """Every head of a full-size workload against the oracle, which compares
    each output element as it goes (nothing of the size of the output is kept
    in float64). Per-head eps is reported; the bar is the global eps."""
    d = make_prefill_inputs(workload)
    if log_gamma is not None:
        d["log_gamma"] = log_gamma
    s0 = d["s0"]
    say("%s N=%d chunk=%d, oracle on all %d heads" % (workload, d["N"], chunk, d["H"]))
    out, st = gpu_prefill(gret, d, chunk, s0)
    _, s_ref, stats = oracle.oracle_prefill_f64(d["q"], d["k"], d["v"], d["log_gamma"], s0,
                                                want_out=False, compare=out)
    e_o, e_s = stats_eps(stats), eps(st, s_ref)
    per_head = stats[:, 0] / stats[:, 1]
    say("   eps_out=%.3e eps_state=%.3e per-head eps max %.3e (head %d) min %.3e" % (
        e_o, e_s, per_head.max(), int(per_head.argmax()), per_head.min()))
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16
    if first_chunk:
        # the initial state decays within a few hundred positions; its effect
        # is checked on its own over the first chunk of every head
        n = chunk
        o_ref, _, _ = oracle.oracle_prefill_f64(
            np.ascontiguousarray(d["q"][:, :, :n]), np.ascontiguousarray(d["k"][:, :, :n]),
            np.ascontiguousarray(d["v"][:, :, :n]),
            np.ascontiguousarray(d["log_gamma"][:, :, :n]), s0)
        e_f = eps(out[:, :, :n], o_ref)
        say("   first-chunk eps=%.3e" % e_f)
        assert e_f <= TOL_BF16


@pytest.mark.timeout(900)
def test_prefill_512k_all_heads(gret):
    _full_check(gret, "prefill_512k", 64)


@pytest.mark.timeout(900)
def test_prefill_1m_all_heads(gret):
    _full_check(gret, "prefill_1m", 64, first_chunk=True)


@pytest.mark.timeout(900)
def test_prefill_512k_slow_decay_all_heads(gret):
    """The 512K workload with gates near 1 (u ~ N(4, 1): mean log-gate about
    -0.0018), where a segment's incoming state stays alive over most of the
    segment and the schedule recomputes the most."""
    cfg = CONFIGS["prefill_512k"]
    lg = slow_decay_log_gamma(cfg["B"], cfg["H"], cfg["N"])
    _full_check(gret, "prefill_512k", 64, log_gamma=lg)


# ------------------------------------------- one head longer than 2^23 rows

@pytest.mark.timeout(900)
def test_prefill_head_longer_than_2_pow_23(gret):
    """One head of 2^23 + 2^21 + 37 rows (past any 32-bit byte offset of the
    head's own rows): the plain prefill at chunk 64 and 256 and the gated
    prefill, inputs drawn on the device by a seeded generator (log-gates by the
    workloads' gate map). The first 4096 rows are checked against the oracle
    over the whole prefix. Sampled rows after that (around 2^23, at segment
    starts, the last rows and 160 random ones) and the final state are checked
    against the oracle over the 2048 rows ending at each, from a zero state:
    the state carried into such a window reaches its last row only through
    exp(sum of the window's later log-gates), which the test checks is below
    exp(-60), far under the bf16 tolerance."""
    from workloads import gate_log_gamma

    N, d, W = (1 << 23) + (1 << 21) + 37, 128, 2048
    say("prefill one head N=%d d=%d" % (N, d))
    g = torch.Generator(device="cuda").manual_seed(2323)
    qd = (torch.randn((1, 1, N, d), generator=g, device="cuda") * d ** -0.5).to(torch.bfloat16)
    kd = (torch.randn((1, 1, N, d), generator=g, device="cuda") * d ** -0.5).to(torch.bfloat16)
    vd = torch.randn((1, 1, N, d), generator=g, device="cuda").to(torch.bfloat16)
    lg = gate_log_gamma(torch.randn((N,), generator=g, device="cuda").cpu().numpy())
    lgd = torch.from_numpy(lg).cuda().view(1, 1, N)
    gate = (2.0 * torch.randn((1, 1, N, d), generator=g, device="cuda")).to(torch.bfloat16)

    # rows to check: window ends (a segment of the launch starts at chunk
    # g * nc // 256 of the head on a 256-CU GPU)
    rng = np.random.default_rng(23)
    nc = (N + 63) // 64
    starts = [(gg * nc // 256) * 64 for gg in (1, 2, 100, 200, 255)]
    ends = np.unique(np.concatenate([
        [4096, (1 << 23) - 1, 1 << 23, (1 << 23) + 1, N - 2, N - 1],
        [r for p in starts for r in (p - 1, p, p + 1)],
        rng.integers(4096, N, 160)]))
    win = ends[:, None] - (W - 1) + np.arange(W)[None, :]   # [samples, W] rows
    rows = np.unique(win.ravel())
    at = np.searchsorted(rows, win)
    ti = torch.from_numpy(rows).cuda()
    hq, hk, hv = (to_host(t[0, 0, ti].contiguous()) for t in (qd, kd, vd))
    wq, wk, wv = (np.ascontiguousarray(a[at])[None] for a in (hq, hk, hv))
    wl = np.ascontiguousarray(lg[win])[None]
    decay = wl[0, :, 1:].astype(np.float64).sum(axis=1)
    assert decay.max() < -60.0, decay.max()
    o_w, s_w, _ = oracle.oracle_prefill_f64(wq, wk, wv, wl)   # one window per oracle head
    o_ref, s_ref = o_w[0, :, -1], s_w[0, -1]                  # the last window ends at N - 1
    o0, _, _ = oracle.oracle_prefill_f64(
        to_host(qd[:, :, :4096].contiguous()), to_host(kd[:, :, :4096].contiguous()),
        to_host(vd[:, :, :4096].contiguous()), lg[None, None, :4096].copy())
    eti = torch.from_numpy(ends).cuda()
    y_ref = oracle_output_gate_f64(o_ref[None, None], to_host(gate[0, 0, eti].contiguous())[None, None])
    y0 = oracle_output_gate_f64(o0, to_host(gate[:, :, :4096].contiguous()))
    for chunk, gated in ((64, False), (256, False), (64, True)):
        if gated:
            out, st = gret.gret_prefill_gated(qd, kd, vd, lgd, gate, chunk=chunk)
        else:
            out, st = gret.gret_prefill(qd, kd, vd, lgd, None, chunk=chunk)
        torch.cuda.synchronize()
        e_o = eps(to_host(out[0, 0, eti].contiguous())[None, None], y_ref if gated else o_ref[None, None])
        e_0 = eps(to_host(out[:, :, :4096].contiguous()), y0 if gated else o0)
        e_s = eps(to_host(st)[0, 0], s_ref)
        say("   chunk %d%s: %d sampled rows eps=%.3e, first 4096 rows eps=%.3e, state eps=%.3e"
            % (chunk, " gated" if gated else "", len(ends), e_o, e_0, e_s))
        assert e_o <= TOL_BF16 and e_0 <= TOL_BF16 and e_s <= TOL_BF16, (chunk, gated, e_o, e_0, e_s)
        del out, st
    del qd, kd, vd, gate, lgd
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128), (128, 128)])
def test_decode_small(gret, dtype, dk, dv):
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    d, S0 = small_inputs(3, 5, 6, dk, dv, dtype=dtype, seed=dk * 3 + dv)
    state = to_dev(S0)
    s64 = S0.astype(np.float64)
    for t in range(6):
        args = [np.ascontiguousarray(d[key][:, :, t]) for key in ("q", "k", "v", "log_gamma")]
        o = gret.gret_decode_step(*(to_dev(a) for a in args), state)
        torch.cuda.synchronize()
        o_r = oracle.oracle_decode_f64(*args, s64)
        assert eps(to_host(o), o_r) <= tol
    assert eps(to_host(state), s64) <= tol
    # zero initial state, separate output state
    args = [np.ascontiguousarray(d[key][:, :, 0]) for key in ("q", "k", "v", "log_gamma")]
    so = torch.empty_like(state)
    o = gret.gret_decode_step(*(to_dev(a) for a in args), None, state_out=so)
    torch.cuda.synchronize()
    z = np.zeros_like(s64)
    o_r = oracle.oracle_decode_f64(*args, z)
    assert eps(to_host(o), o_r) <= tol and eps(to_host(so), z) <= tol


@pytest.mark.timeout(900)
def test_decode_b256_1000_steps_all_heads(gret):
    cfg = CONFIGS["decode_b256"]
    B, H, steps = cfg["B"], cfg["H"], cfg["decode_steps"]
    say("decode_b256 B=%d H=%d steps=%d, oracle on all heads and steps" % (B, H, steps))
    d = make_decode_inputs("decode_b256")
    state = to_dev(d["state"])
    q, k, v, lg = (to_dev(d[key]) for key in ("q", "k", "v", "log_gamma"))
    outs = torch.empty((steps, B, H, 128), dtype=torch.bfloat16, device="cuda")
    for t in range(steps):
        gret.gret_decode_step(q[t], k[t], v[t], lg[t], state, out=outs[t])
    torch.cuda.synchronize()
    outs = to_host(outs)
    st = to_host(state)
    s64 = d["state"].astype(np.float64)
    worst, worst_t = 0.0, -1
    for t in range(steps):
        o_r = oracle.oracle_decode_f64(d["q"][t], d["k"][t], d["v"][t], d["log_gamma"][t], s64)
        e = eps(outs[t], o_r)
        if e > worst:
            worst, worst_t = e, t
    e_s = eps(st, s64)
    say("   worst per-step eps=%.3e (step %d) final-state eps=%.3e" % (worst, worst_t, e_s))
    assert worst <= TOL_BF16 and e_s <= TOL_BF16


if __name__ == "__main__":  # pragma: no cover
    sys.exit(pytest.main([os.path.abspath(__file__), "-x", "-v", "-m", "gpu"]))
