"""The library holds no global state and is reentrant (include/gret.h): calls
on different HIP streams that run at the same time must give exactly the
results of the same calls made one after another.

A prefill, a run of decode steps, a cross-attention decode and a projection are
each launched on their own stream (default priority), all before any of them
is waited for, and every output is compared bit for bit with a sequential run
on the default stream. The kernels are deterministic (fixed reduction orders,
no atomics), so any difference would be interference between calls.
"""
import numpy as np
import pytest
import torch

from tests.gpu_util import to_dev
from workloads import (make_attention_inputs, make_decode_inputs, make_prefill_inputs,
                       make_projection_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gret():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import yoco_gated_retention_amd as g

    g.load_library()
    return g


def _inputs():
    p = make_prefill_inputs("prefill_32k", N=3000, H=6)
    d = make_decode_inputs("decode_b256", B=8, H=6, steps=5)
    q, k, v = make_attention_inputs(41, 2, 8, 2, 5000, 128)
    x, wk, wg = make_projection_inputs(42, 1, 1500, 512, 4, 128)
    dev = {
        "pq": to_dev(p["q"]), "pk": to_dev(p["k"]), "pv": to_dev(p["v"]),
        "plg": to_dev(p["log_gamma"]),
        "ds0": to_dev(d["state"]), "dq": to_dev(d["q"]), "dk": to_dev(d["k"]),
        "dv": to_dev(d["v"]), "dlg": to_dev(d["log_gamma"]),
        "xq": to_dev(q[:, :, -1].copy()), "xk": to_dev(k), "xv": to_dev(v),
        "x": to_dev(x), "wk": to_dev(wk), "wg": to_dev(wg),
    }
    return dev


def _run_all(gret, t, streams):
    """Launches the four calls, each on its stream, without waiting between
    them. Returns the output tensors (not yet synchronized)."""
    res = {}
    with torch.cuda.stream(streams[0]):
        res["prefill"] = gret.gret_prefill(t["pq"], t["pk"], t["pv"], t["plg"], None, chunk=64)
    with torch.cuda.stream(streams[1]):
        state = t["ds0"].clone()
        outs = []
        for s in range(t["dq"].shape[0]):
            outs.append(gret.gret_decode_step(t["dq"][s], t["dk"][s], t["dv"][s], t["dlg"][s],
                                              state))
        res["decode"] = (torch.stack(outs), state)
    with torch.cuda.stream(streams[2]):
        res["xattn"] = (gret.gret_cross_attention_decode(t["xq"], t["xk"], t["xv"]),)
    with torch.cuda.stream(streams[3]):
        res["proj"] = gret.gret_head_projection(t["x"], t["wk"], t["wg"], key_scale=0.125,
                                                temperature=16.0)
    return res


def test_concurrent_streams_match_sequential(gret):
    t = _inputs()
    torch.cuda.synchronize()
    default = torch.cuda.current_stream()
    seq = _run_all(gret, t, [default] * 4)
    torch.cuda.synchronize()
    seq = {k: tuple(x.clone() for x in v) for k, v in seq.items()}

    streams = [torch.cuda.Stream() for _ in range(4)]
    for s in streams:
        s.wait_stream(default)
    for rep in range(3):
        par = _run_all(gret, t, streams)
        for s in streams:
            default.wait_stream(s)
        torch.cuda.synchronize()
        for name, outs in par.items():
            for i, (a, b) in enumerate(zip(outs, seq[name])):
                same = torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                                   b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
                assert same, "%s output %d differs on concurrent streams (repeat %d)" % (
                    name, i, rep)
    assert np.isfinite(seq["prefill"][0].float().cpu().numpy()).all()
