"""The Python binding rejects caller-supplied buffers of the wrong shape before
any library call (CPU only: no GPU, and the library is replaced by a recorder
that fails the test if anything is called).

The kernels take every size from q and v (and the caches or rings), so an
undersized out, state or ring buffer must never reach them."""
import pytest
import torch

import yoco_gated_retention_amd as gret


class _Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return 0
        return fn


@pytest.fixture
def rec(monkeypatch):
    r = _Recorder()
    monkeypatch.setattr(gret, "_lib", r)
    return r


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


B, H, N, DK, DV = 2, 3, 100, 64, 128


def prefill_args():
    return dict(q=bf(B, H, N, DK), k=bf(B, H, N, DK), v=bf(B, H, N, DV), log_gamma=f32(B, H, N))


@pytest.mark.parametrize("name,bad", [
    ("out", bf(B, H, N - 1, DV)), ("out", bf(B, H, N, DK)), ("state_out", f32(B, H, DK, DK)),
    ("state_in", f32(B, H, DV, DK)), ("state_in", f32(1, H, DK, DV)),
])
def test_prefill_rejects_wrong_buffer_shapes(rec, name, bad):
    with pytest.raises(ValueError, match="%s must have shape" % name):
        gret.gret_prefill(**prefill_args(), **{name: bad})
    assert rec.calls == []


def test_prefill_rejects_wrong_input_shapes(rec):
    a = prefill_args()
    with pytest.raises(ValueError, match="k must have shape"):
        gret.gret_prefill(a["q"], bf(B, H, N, DK + 64), a["v"], a["log_gamma"])
    with pytest.raises(ValueError, match="log_gamma must have shape"):
        gret.gret_prefill(a["q"], a["k"], a["v"], f32(B, H, N + 1))
    with pytest.raises(ValueError):
        gret.gret_prefill(a["q"], a["k"], bf(B, H, N + 1, DV), a["log_gamma"])
    assert rec.calls == []


@pytest.mark.parametrize("name,bad", [
    ("gate", bf(B, H, N, DK)), ("norm_weight", f32(H, DK)), ("norm_bias", f32(H + 1, DV)),
])
def test_prefill_gated_rejects_wrong_shapes(rec, name, bad):
    kw = dict(gate=bf(B, H, N, DV))
    kw[name] = bad
    with pytest.raises(ValueError, match="%s must have shape" % name):
        gret.gret_prefill_gated(**prefill_args(), **kw)
    assert rec.calls == []


def test_prefill_right_shapes_still_need_a_gpu(rec):
    # correct shapes pass the shape stage; CPU tensors are then refused
    with pytest.raises(ValueError, match="GPU tensor"):
        gret.gret_prefill(**prefill_args(), out=bf(B, H, N, DV), state_out=f32(B, H, DK, DV))
    assert rec.calls == []


@pytest.mark.parametrize("name,bad", [
    ("out", bf(B, H, DK)), ("state_out", f32(B, H, DK, DK)), ("state_in", f32(B, H + 1, DK, DV)),
])
def test_decode_rejects_wrong_buffer_shapes(rec, name, bad):
    kw = dict(q=bf(B, H, DK), k=bf(B, H, DK), v=bf(B, H, DV), log_gamma=f32(B, H),
              state_in=f32(B, H, DK, DV))
    kw[name] = bad
    with pytest.raises(ValueError, match="%s must have shape" % name):
        gret.gret_decode_step(**kw)
    with pytest.raises(ValueError, match="%s must have shape" % name):
        gret.gret_decode_step_gated(**kw, gate=bf(B, H, DV))
    assert rec.calls == []


def test_decode_in_place_state_shape_checked(rec):
    # state_out defaults to state_in, which must then have the state's shape
    with pytest.raises(ValueError, match="must have shape"):
        gret.gret_decode_step(bf(B, H, DK), bf(B, H, DK), bf(B, H, DV), f32(B, H),
                              f32(B, H, DK, DV - 1))
    assert rec.calls == []


@pytest.mark.parametrize("name,bad", [
    ("out", bf(2, 8, 63)), ("v_cache", bf(2, 2, 500, 64)), ("lengths", torch.zeros(3, dtype=torch.int32)),
])
def test_cross_attention_rejects_wrong_shapes(rec, name, bad):
    kw = dict(q=bf(2, 8, 64), k_cache=bf(2, 2, 512, 64), v_cache=bf(2, 2, 512, 64))
    kw[name] = bad
    with pytest.raises(ValueError, match="%s must have shape" % name):
        gret.gret_cross_attention_decode(**kw)
    assert rec.calls == []


@pytest.mark.parametrize("name,bad", [("k_out", bf(1, 2, 10, 32)), ("log_gamma", f32(1, 2, 9))])
def test_projection_rejects_wrong_shapes(rec, name, bad):
    kw = dict(x=bf(1, 10, 128), w_key=bf(2 * 64, 128), w_gamma=bf(2, 128))
    kw[name] = bad
    with pytest.raises(ValueError, match="%s must have shape" % name):
        gret.gret_head_projection(**kw)
    assert rec.calls == []


@pytest.mark.parametrize("name,bad", [
    ("out", bf(1, 4, 99, 64)), ("k_ring", bf(1, 2, 32, 64)), ("v_ring", bf(1, 2, 64, 32)),
])
def test_swa_prefill_rejects_wrong_shapes(rec, name, bad):
    kw = dict(q=bf(1, 4, 100, 64), k=bf(1, 2, 100, 64), v=bf(1, 2, 100, 64), window=64,
              k_ring=bf(1, 2, 64, 64), v_ring=bf(1, 2, 64, 64))
    kw[name] = bad
    with pytest.raises(ValueError, match="%s must have shape" % name):
        gret.gret_swa_prefill(**kw)
    assert rec.calls == []


@pytest.mark.parametrize("name,bad", [
    ("out", bf(3, 4, 32)), ("v_ring", bf(3, 2, 63, 64)), ("k_new", bf(3, 4, 64)),
    ("positions", torch.zeros(2, dtype=torch.int32)),
])
def test_swa_decode_rejects_wrong_shapes(rec, name, bad):
    kw = dict(q=bf(3, 4, 64), k_new=bf(3, 2, 64), v_new=bf(3, 2, 64), k_ring=bf(3, 2, 64, 64),
              v_ring=bf(3, 2, 64, 64), positions=torch.zeros(3, dtype=torch.int32))
    kw[name] = bad
    with pytest.raises(ValueError, match="%s must have shape" % name):
        gret.gret_swa_decode_step(**kw)
    assert rec.calls == []
