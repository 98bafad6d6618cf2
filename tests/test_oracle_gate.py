"""Pins for the fp64 output-epilogue oracle (GroupNorm per head + swish gate).

The definition follows the page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV
Cache 只存一次", section "路线二：Multi-Head Gated Retention" (per-head
normalisation of the multi-head output, then the element-wise gate
swish(X W_G)). The oracle is checked against a hand-worked example, against the
library routines torch.nn.functional.group_norm (one group per head) and silu,
and against invariances that GroupNorm must have.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle_output_gate_f64
from workloads import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "output_gate_worked_example.txt")


def _golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, *rest = line.split()
            vals[name] = np.array([float(x) for x in rest])
    return vals


@pytest.mark.parametrize("affine", [False, True])
def test_worked_example(affine):
    g = _golden()
    o = g["o"].reshape(1, 1, 1, 4)
    gate = np.log(g["gate_ln_arg"]).reshape(1, 1, 1, 4)
    w = g["weight"].reshape(1, 4) if affine else None
    b = g["bias"].reshape(1, 4) if affine else None
    y = oracle_output_gate_f64(o, gate, w, b, eps=float(g["eps"][0]))
    z = g["z_affine"] if affine else g["z"]
    want = np.log(g["gate_ln_arg"]) * g["sigmoid"] * z
    np.testing.assert_allclose(y.reshape(-1), want, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("shape", [(2, 3, 5, 64), (1, 4, 7, 128), (3, 2, 16)])
@pytest.mark.parametrize("affine", [False, True])
def test_matches_torch_group_norm_and_silu(shape, affine):
    rng = np.random.default_rng(7)
    o = rng.standard_normal(shape) * 3.0 + 0.7
    gate = rng.standard_normal(shape) * 2.0
    H, dv = shape[1], shape[-1]
    w = rng.standard_normal((H, dv)) if affine else None
    b = rng.standard_normal((H, dv)) if affine else None
    y = oracle_output_gate_f64(o, gate, w, b, eps=1e-5)
    # torch: rows = every (batch, position), channels = H * dv, one group per head
    t = torch.from_numpy(np.moveaxis(o, 1, -2).reshape(-1, H * dv))
    tw = torch.from_numpy(w.reshape(-1)) if affine else None
    tb = torch.from_numpy(b.reshape(-1)) if affine else None
    gn = torch.nn.functional.group_norm(t, H, tw, tb, eps=1e-5)
    gt = torch.from_numpy(np.moveaxis(gate, 1, -2).reshape(-1, H * dv))
    ref = (torch.nn.functional.silu(gt) * gn).numpy()
    ref = np.moveaxis(ref.reshape(np.moveaxis(o, 1, -2).shape), -2, 1)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_shift_and_scale_invariance():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((2, 3, 9, 32))
    gate = rng.standard_normal(o.shape)
    y0 = oracle_output_gate_f64(o, gate, eps=0.0)
    y1 = oracle_output_gate_f64(o * 37.5 - 11.0, gate, eps=0.0)
    np.testing.assert_allclose(y1, y0, rtol=1e-10, atol=1e-11)


def test_normalised_rows_have_zero_mean_unit_variance():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((1, 2, 6, 64)) * 5 + 2
    # with gate = ln 3 everywhere, swish(gate) = (3/4) ln 3 exactly
    gate = np.full(o.shape, math.log(3.0))
    z = oracle_output_gate_f64(o, gate, eps=0.0) / (0.75 * math.log(3.0))
    np.testing.assert_allclose(z.mean(axis=-1), 0.0, atol=1e-12)
    np.testing.assert_allclose((z ** 2).mean(axis=-1), 1.0, rtol=1e-12)


def test_zero_gate_and_constant_rows():
    o = np.arange(2 * 3 * 4 * 8, dtype=np.float64).reshape(2, 3, 4, 8)
    assert np.all(oracle_output_gate_f64(o, np.zeros_like(o)) == 0.0)
    c = np.full((1, 2, 3, 16), 4.25)
    # constant row: deviations are exactly 0, so the output is the bias times the gate
    bias = np.arange(32, dtype=np.float64).reshape(2, 16)
    y = oracle_output_gate_f64(c, np.full(c.shape, math.log(7.0)), None, bias, eps=1e-5)
    want = np.broadcast_to(math.log(7.0) * 0.875 * bias.reshape(1, 2, 1, 16), c.shape)
    np.testing.assert_allclose(y, want, rtol=1e-14)


def test_affine_is_per_head():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((1, 3, 4, 16))
    gate = rng.standard_normal(o.shape)
    w = rng.standard_normal((3, 16))
    b = rng.standard_normal((3, 16))
    y = oracle_output_gate_f64(o, gate, w, b)
    perm = [2, 0, 1]
    yp = oracle_output_gate_f64(o[:, perm], gate[:, perm], w[perm], b[perm])
    np.testing.assert_allclose(yp, y[:, perm], rtol=0, atol=0)


def test_bf16_inputs_are_widened_exactly():
    rng = np.random.default_rng(6)
    o32 = rng.standard_normal((1, 2, 3, 64)).astype(np.float32)
    g32 = rng.standard_normal(o32.shape).astype(np.float32)
    ob, gb = f32_to_bf16_bits(o32), f32_to_bf16_bits(g32)
    widened_o = (ob.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    widened_g = (gb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(oracle_output_gate_f64(ob, gb),
                                  oracle_output_gate_f64(widened_o, widened_g))
