"""gret_prefill_noalloc (the library's fixed device scratch in place of the
caller's workspace) against gret_prefill, through the C ABI.

Both entry points run the same kernels on the same segment plan, so their
outputs and final states must agree bit for bit (stricter than the parity bar
of 1e-2 for bf16 and 1e-4 for fp32, which is also checked against the fp64
oracle). Two calls in a row, the second one smaller, check that what the
first call left in the scratch does not leak into the second.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import eps, to_dev, to_host
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

SCRATCH_ERR = 8


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import yoco_gated_retention_amd as g

    oracle.build_oracle(force=False)
    return g.load_library()


def inputs(B, H, N, dk, dv, dtype, seed, s0=True):
    rng = np.random.default_rng(seed)

    def st(x):
        return f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)

    d = dict(q=st(rng.standard_normal((B, H, N, dk), dtype=np.float32) / np.sqrt(dk)),
             k=st(rng.standard_normal((B, H, N, dk), dtype=np.float32) / np.sqrt(dk)),
             v=st(rng.standard_normal((B, H, N, dv), dtype=np.float32)),
             log_gamma=(-np.logaddexp(0.0, -rng.standard_normal((B, H, N))) / 16.0
                        ).astype(np.float32))
    S0 = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32) if s0 else None
    return d, S0


def vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def run_both(lib, d, S0, chunk):
    q, k, v, lg = (to_dev(d[x]) for x in ("q", "k", "v", "log_gamma"))
    si = None if S0 is None else to_dev(S0)
    B, H, N, dk = q.shape
    dv = v.shape[3]
    code = 1 if q.dtype == torch.bfloat16 else 0
    out_a, out_b = torch.empty((B, H, N, dv), dtype=q.dtype, device="cuda"), None
    out_b = torch.empty_like(out_a)
    st_a = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    st_b = torch.empty_like(st_a)
    need = ctypes.c_size_t(0)
    assert lib.gret_prefill_workspace_bytes(B, H, N, dk, dv, chunk, code, ctypes.byref(need)) == 0
    ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device="cuda")
    rc = lib.gret_prefill(vp(q), vp(k), vp(v), vp(lg), vp(si), vp(out_a), vp(st_a), B, H, N, dk,
                          dv, chunk, code, vp(ws), need.value, stream())
    assert rc == 0, rc
    rc = lib.gret_prefill_noalloc(vp(q), vp(k), vp(v), vp(lg), vp(si), vp(out_b), vp(st_b), B, H,
                                  N, dk, dv, chunk, code, stream())
    assert rc == 0, rc
    torch.cuda.synchronize()
    return to_host(out_a), to_host(st_a), to_host(out_b), to_host(st_b)


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_noalloc_matches_workspace_entry_two_calls(lib, chunk):
    tol = 1e-2
    # first call: all 24 heads of a long prompt; second: fewer, shorter heads
    for (B, H, N, dk, dv, seed) in ((1, 24, 40000, 128, 128, 11), (2, 3, 1777, 64, 128, 12)):
        say("noalloc chunk=%d B=%d H=%d N=%d dk=%d dv=%d" % (chunk, B, H, N, dk, dv))
        d, S0 = inputs(B, H, N, dk, dv, "bf16", seed + chunk)
        oa, sa, ob, sb = run_both(lib, d, S0, chunk)
        assert np.array_equal(oa, ob) and np.array_equal(sa, sb)
        _, s_ref, stats = oracle.oracle_prefill_f64(d["q"], d["k"], d["v"], d["log_gamma"], S0,
                                                    want_out=False, compare=ob)
        e_o = float(np.max(stats[:, 0]) / np.max(stats[:, 1]))
        e_s = eps(sb, s_ref)
        say("   bitwise equal; eps_out=%.3e eps_state=%.3e" % (e_o, e_s))
        assert e_o <= tol and e_s <= tol


def test_noalloc_fp32_path(lib):
    d, S0 = inputs(1, 2, 700, 64, 64, "f32", 21)
    oa, sa, ob, sb = run_both(lib, d, S0, 64)
    assert np.array_equal(oa, ob) and np.array_equal(sa, sb)
    o_ref, s_ref, _ = oracle.oracle_prefill_f64(d["q"], d["k"], d["v"], d["log_gamma"], S0)
    assert eps(ob, o_ref) <= 1e-4 and eps(sb, s_ref) <= 1e-4


def test_noalloc_rejects_requests_beyond_the_scratch(lib):
    # 4096 heads of 64 KiB segment states cannot fit 64 MiB: refused before
    # anything is enqueued (the output keeps its sentinel)
    B, H, N, dk, dv = 4096, 1, 64, 128, 128
    q = torch.zeros((B, H, N, dk), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
    out = torch.full((B, H, N, dv), 7.0, dtype=torch.bfloat16, device="cuda")
    st = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    rc = lib.gret_prefill_noalloc(vp(q), vp(q), vp(q), vp(lg), None, vp(out), vp(st), B, H, N,
                                  dk, dv, 64, 1, stream())
    torch.cuda.synchronize()
    assert rc == SCRATCH_ERR
    assert bool((out == 7.0).all())
