"""The entry points allocate nothing, synchronise nothing and enqueue only
kernels on the caller's stream, so a caller can capture them in a HIP graph
and replay it (a serving loop's decode step, for instance).

Each test captures calls with preallocated outputs and workspace, then replays
the graph several times with new inputs copied into its static buffers, with
eager work and a synchronisation between replays, and compares every replay
bit for bit with the same call made eagerly.
"""
import pytest
import torch

from tests.gpu_util import to_dev
from workloads import make_attention_inputs, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gret():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import yoco_gated_retention_amd as g

    g.load_library()
    return g


def _same(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def test_decode_and_cross_attention_replay(gret):
    steps = 5
    d = make_decode_inputs("decode_b256", B=16, H=6, steps=steps)
    dq, dk, dv, dlg = (to_dev(d[n]) for n in ("q", "k", "v", "log_gamma"))
    s0 = to_dev(d["state"])
    q, k, v = make_attention_inputs(7, 4, 12, 3, 3000, 128)
    xq_all, xk, xv = to_dev(q[:, :, :steps].transpose(2, 0, 1, 3).copy()), to_dev(k), to_dev(v)
    # static buffers of the graph
    sq, sk, sv, slg = dq[0].clone(), dk[0].clone(), dv[0].clone(), dlg[0].clone()
    state = s0.clone()
    out = torch.empty((16, 6, 128), dtype=torch.bfloat16, device="cuda")
    sxq = xq_all[0].clone()
    ws = torch.empty(gret.gret_cross_attention_workspace_bytes(4, 12, 3, 3000, 128),
                     dtype=torch.uint8, device="cuda")
    xout = torch.empty((4, 12, 128), dtype=torch.bfloat16, device="cuda")

    def calls():
        gret.gret_decode_step(sq, sk, sv, slg, state, out=out)
        gret.gret_cross_attention_decode(sxq, xk, xv, out=xout, workspace=ws)

    # warm up eagerly (library loaded, kernels resident), then restore the state
    calls()
    torch.cuda.synchronize()
    state.copy_(s0)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    state.copy_(s0)

    ref_state = s0.clone()
    for s in range(steps):
        for dst, src in ((sq, dq), (sk, dk), (sv, dv), (slg, dlg), (sxq, xq_all)):
            dst.copy_(src[s])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_out = gret.gret_decode_step(dq[s], dk[s], dv[s], dlg[s], ref_state)
        ref_x = gret.gret_cross_attention_decode(xq_all[s], xk, xv)
        torch.cuda.synchronize()
        assert _same(out, ref_out), "decode replay %d" % s
        assert torch.equal(state, ref_state), "decode state replay %d" % s
        assert _same(xout, ref_x), "cross-attention replay %d" % s


def test_prefill_replay(gret):
    p = make_prefill_inputs("prefill_32k", N=2000, H=4)
    q, k, v, lg = (to_dev(p[n]) for n in ("q", "k", "v", "log_gamma"))
    B, H, N, dk = q.shape
    dv = v.shape[3]
    assert gret.gret_prefill_workspace_bytes(B, H, N, dk, dv, 64, q.dtype) > 0, \
        "this shape should take the segment-parallel path, which uses the workspace"
    sq, sk, sv, slg = q.clone(), k.clone(), v.clone(), lg.clone()
    out = torch.empty((B, H, N, dv), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, gret.gret_prefill_workspace_bytes(B, H, N, dk, dv, 64, q.dtype)),
                     dtype=torch.uint8, device="cuda")

    def call():
        gret.gret_prefill(sq, sk, sv, slg, None, chunk=64, out=out, state_out=st, workspace=ws)

    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        # a different prompt each replay: rotate the heads
        perm = [(h + rep) % H for h in range(H)]
        for dst, src in ((sq, q), (sk, k), (sv, v), (slg, lg)):
            dst.copy_(src[:, perm])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_out, ref_st = gret.gret_prefill(q[:, perm].contiguous(), k[:, perm].contiguous(),
                                            v[:, perm].contiguous(), lg[:, perm].contiguous(),
                                            None, chunk=64)
        torch.cuda.synchronize()
        assert _same(out, ref_out), "prefill replay %d" % rep
        assert torch.equal(st, ref_st), "prefill state replay %d" % rep
