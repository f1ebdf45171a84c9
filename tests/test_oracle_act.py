"""Pins for the oracle's parameterised expert activation (CPU only).

The pages leave the released model's activation open; the oracle reads it as a SwiGLU with
optional interleaved gate/up rows, a clamp (gate from above only, up on both sides), a sigmoid
scale alpha, a shift added to up and fp32 biases on both products, such that zero parameters give
the plain SwiGLU. These tests pin it without retyping its formula: equivalences (defaults ==
plain SwiGLU, interleaved rows == halves, u + shift), clamp invariants (every value past the
limit acts as the limit), closed forms where the sigmoid is exactly 3/4 or 1, and the bias's
linearity through the routing weights.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mxfp4_weight_quantized_amd import inputs

RELEASED = dict(alpha=1.702, limit=7.0, up_shift=1.0)


def _layer(seed, T, H, F, E, k):
    x = inputs.activations(seed, T, H)
    w = inputs.expert_weights(seed, E, H, F, oracle.quantize, threads=2)
    r = np.random.default_rng(seed)
    idx = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    wt = r.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    wt /= wt.sum(axis=1, keepdims=True)
    return x, idx, wt, w


def _interleave(a, F):
    """Rows [0, F) gate and [F, 2F) up -> rows 2i gate i, 2i + 1 up i (axis 1)."""
    out = np.empty_like(a)
    out[:, 0::2], out[:, 1::2] = a[:, :F], a[:, F:]
    return out


def test_defaults_are_the_plain_swiglu():
    T, H, F, E, k = 6, 64, 96, 3, 2
    x, idx, wt, (gp, gs, dp, ds) = _layer(41, T, H, F, E, k)
    plain = oracle.moe_mlp(x, idx, wt, gp, gs, dp, ds, E=E)
    np.testing.assert_array_equal(oracle.moe_mlp(x, idx, wt, gp, gs, dp, ds, E=E, act={}), plain)
    a = oracle.moe_mlp(x, idx, wt, gp, gs, dp, ds, E=E, mx_act=True, fragile_c=4.0)
    b = oracle.moe_mlp(x, idx, wt, gp, gs, dp, ds, E=E, mx_act=True, fragile_c=4.0, act={})
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("mx_act", [False, True])
def test_interleaved_rows_equal_halves(mx_act):
    T, H, F, E, k = 7, 64, 64, 4, 2
    x, idx, wt, (gp, gs, dp, ds) = _layer(42, T, H, F, E, k)
    r = np.random.default_rng(42)
    gb = r.normal(0, 0.5, (E, 2 * F)).astype(np.float32)
    db = r.normal(0, 0.5, (E, H)).astype(np.float32)
    half = oracle.moe_mlp(x, idx, wt, gp, gs, dp, ds, E=E, mx_act=mx_act,
                          act=dict(RELEASED, gu_bias=gb, dn_bias=db))
    inter = oracle.moe_mlp(x, idx, wt, _interleave(gp, F), _interleave(gs, F), dp, ds, E=E,
                           mx_act=mx_act, act=dict(RELEASED, interleaved=True,
                                                   gu_bias=_interleave(gb, F), dn_bias=db))
    np.testing.assert_array_equal(inter, half)
    # and the parameters do change the result
    assert np.abs(half - oracle.moe_mlp(x, idx, wt, gp, gs, dp, ds, E=E, mx_act=mx_act)).max() > 0


def _bias_only_layer(gu_pairs, H=32, F=32):
    """Experts whose gate_up weights are all zero, so a = gu_bias: expert e has gate value g and
    up value u (in every column) from gu_pairs[e]; every down row m has 1.0 at f = m."""
    E = len(gu_pairs)
    gp = np.zeros((E, 2 * F, H // 2), np.uint8)
    gs = np.full((E, 2 * F, H // 32), 127, np.uint8)
    codes = np.zeros((H, F), np.uint8)
    codes[np.arange(H), np.arange(H) % F] = 2          # code 2 = 1.0
    dp = np.stack([(codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)] * E)
    ds = np.full((E, H, F // 32), 127, np.uint8)
    gb = np.zeros((E, 2 * F), np.float32)
    for e, (g, u) in enumerate(gu_pairs):
        gb[e, :F], gb[e, F:] = g, u
    x = inputs.activations(43, E, H)
    idx = np.arange(E, dtype=np.int32).reshape(E, 1)  # token e -> expert e
    w = np.ones((E, 1), np.float32)
    return x, idx, w, gp, gs, dp, ds, gb


def test_clamp_acts_as_the_limit_gate_above_only():
    pairs = [(10.0, 0.5), (20.0, 0.5),      # gate above the limit: both act as 4
             (-10.0, 0.5), (-20.0, 0.5),    # gate below -limit: not clamped
             (2.0, 10.0), (2.0, 20.0),      # up above: both 4
             (2.0, -10.0), (2.0, -20.0),    # up below: both -4
             (3.0, 0.5), (3.0, -0.5)]       # inside: untouched
    x, idx, w, gp, gs, dp, ds, gb = _bias_only_layer(pairs)
    E = len(pairs)
    out, h = oracle.moe_mlp(x, idx, w, gp, gs, dp, ds, E=E, want_h=True,
                            act=dict(alpha=1.0, limit=4.0, up_shift=0.0, gu_bias=gb))
    np.testing.assert_array_equal(out[0], out[1])
    assert np.all(out[2] != out[3])
    np.testing.assert_array_equal(out[4], out[5])
    np.testing.assert_array_equal(out[6], out[7])
    assert np.all(out[4] == -out[6])               # u = +4 vs u = -4, same gate
    # inside the limit the clamp changes nothing
    unclamped = oracle.moe_mlp(x, idx, w, gp, gs, dp, ds, E=E, act=dict(gu_bias=gb))
    np.testing.assert_array_equal(out[8:], unclamped[8:])
    assert not np.array_equal(out[:2], unclamped[:2])


def test_shift_is_added_to_up():
    x, idx, w, gp, gs, dp, ds, gb0 = _bias_only_layer([(1.5, 0.0), (-0.75, 0.0)])
    _, _, _, _, _, _, _, gb1 = _bias_only_layer([(1.5, 1.0), (-0.75, 1.0)])
    a = oracle.moe_mlp(x, idx, w, gp, gs, dp, ds, E=2, act=dict(alpha=1.702, up_shift=1.0, gu_bias=gb0))
    b = oracle.moe_mlp(x, idx, w, gp, gs, dp, ds, E=2, act=dict(alpha=1.702, up_shift=0.0, gu_bias=gb1))
    np.testing.assert_array_equal(a, b)
    assert np.all(a != 0)


def test_alpha_closed_forms():
    """alpha g = ln 3 gives sigmoid 3/4; alpha g = 256 gives sigmoid 1 in fp64."""
    g1 = float(np.float32(math.log(3.0) / 2.0))      # the fp32 bias the gate value comes from
    x, idx, w, gp, gs, dp, ds, gb = _bias_only_layer([(g1, 1.0), (4.0, 2.5)])
    _, h = oracle.moe_mlp(x, idx, w, gp, gs, dp, ds, E=2, want_h=True,
                          act=dict(alpha=2.0, gu_bias=gb))
    want0 = torch.tensor(g1 * 0.75 * 1.0, dtype=torch.float64).to(torch.bfloat16).double().item()
    assert np.all(inputs.bf16_to_f32(h[0, 0]) == want0)
    _, h = oracle.moe_mlp(x, idx, w, gp, gs, dp, ds, E=2, want_h=True,
                          act=dict(alpha=64.0, up_shift=1.0, gu_bias=gb))
    assert np.all(inputs.bf16_to_f32(h[1, 0]) == 4.0 * 3.5)     # 4 * 1 * (2.5 + 1)


def test_down_bias_enters_weighted():
    T, H, F, E, k = 5, 64, 64, 3, 3
    x, idx, wt, (gp, gs, dp, ds) = _layer(44, T, H, F, E, k)
    db = np.random.default_rng(44).normal(0, 1.0, (E, H)).astype(np.float32)
    a = oracle.moe_mlp(x, idx, wt, gp, gs, dp, ds, E=E, act=dict(RELEASED, dn_bias=db))
    b = oracle.moe_mlp(x, idx, wt, gp, gs, dp, ds, E=E, act=dict(RELEASED))
    want = np.einsum("tj,tjh->th", wt.astype(np.float64), db.astype(np.float64)[idx])
    np.testing.assert_allclose(a - b, want, rtol=1e-9, atol=1e-12)
