"""Pins for the weight operand of the oracle's matrix products (CPU only).

Reading of the open point (the pages describe the de-quantized model as the bf16 one): with bf16
activations the weight enters the product as the bf16 value of code * 2^(b-127), which is the
exact value except past bf16's largest finite number (+-Inf); the activation variant multiplies
MXFP4 by MXFP4 as they are, with exact values. References: the golden E2M1 table with closed-form
powers of two, torch's bf16 cast, and hand-built packed weights whose products have closed forms.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from mxfp4_weight_quantized_amd import inputs


def _table(golden_dir):
    tab = np.zeros(16)
    with open(os.path.join(golden_dir, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                c, v = line.split()
                tab[int(c, 16)] = float(v)
    return tab


def _pack(codes):
    """codes [R][K] (0..15) -> packed [R][K/2], element 2j in the low nibble of byte j."""
    codes = np.asarray(codes, np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _bf16_bits_exact(v):
    """bf16 bits of a value that bf16 holds exactly (the tests' inputs)."""
    b = inputs.bf16_bits(np.array([v], np.float32))[0]
    assert inputs.bf16_to_f32(np.array([b], np.uint16))[0] == v
    return b


def test_weight_operand_all_codes_and_scale_bytes(golden_dir):
    tab = _table(golden_dir)
    n_inf = 0
    for b in range(256):
        for c in range(16):
            ex = oracle.weight_operand(c, b, mx_act=True)
            bf = oracle.weight_operand(c, b, mx_act=False)
            if b == 255:
                assert math.isnan(ex) and math.isnan(bf)
                continue
            exact = tab[c] * 2.0 ** (b - 127)
            assert ex == exact and math.copysign(1, ex) == math.copysign(1, exact), (b, c)
            want = torch.tensor(exact, dtype=torch.float64).to(torch.bfloat16).double().item()
            assert bf == want and math.copysign(1, bf) == math.copysign(1, want), (b, c, bf, want)
            if math.isinf(bf):
                n_inf += 1
                # only values past bf16's largest finite number (2^128 - 2^120) overflow
                assert abs(exact) > (2.0 ** 128 - 2.0 ** 120) and b in (253, 254)
            else:
                assert bf == exact  # everything else, subnormals included, is exact in bf16
    # byte 253: |code| in {4, 6}; byte 254: |code| in {2, 3, 4, 6}; both signs
    assert n_inf == 2 * (2 + 4)


def test_linear_overflowing_weight_is_inf_on_bf16_path_and_exact_on_fp4_path():
    """One weight element per row: 6 * 2^127 (code 7, byte 254), -6 * 2^127 (code 15) and
    1.5 * 2^127 (code 3); x = 2^-100 at that element. bf16 path: +Inf, -Inf, 1.5 * 2^27.
    Activation variant (x quantized: one nonzero element is exact): 6 * 2^27, -6 * 2^27,
    1.5 * 2^27."""
    K = 32
    codes = np.zeros((3, K), np.uint8)
    codes[0, 0], codes[1, 0], codes[2, 0] = 7, 15, 3
    p = _pack(codes)
    s = np.full((3, 1), 254, np.uint8)
    x = np.zeros((1, K), np.uint16)
    x[0, 0] = _bf16_bits_exact(2.0 ** -100)
    y = oracle.linear(x, p, s)
    assert y[0, 0] == math.inf and y[0, 1] == -math.inf and y[0, 2] == 1.5 * 2.0 ** 27
    ym = oracle.linear(x, p, s, mx_act=True)
    np.testing.assert_array_equal(ym[0], [6 * 2.0 ** 27, -6 * 2.0 ** 27, 1.5 * 2.0 ** 27])


def test_linear_subnormal_weights_are_kept():
    """Byte 0: code 1 is 2^-128, a bf16 subnormal; x = 2^100 at that element gives 2^-28."""
    K = 64
    codes = np.zeros((2, K), np.uint8)
    codes[0, 5] = 1      # 0.5 * 2^-127
    codes[1, 40] = 9     # -0.5 * 2^(1-127), block 1 of row 1 uses byte 1
    p = _pack(codes)
    s = np.array([[0, 0], [0, 1]], np.uint8)
    x = np.zeros((1, K), np.uint16)
    x[0, 5] = _bf16_bits_exact(2.0 ** 100)
    x[0, 40] = _bf16_bits_exact(2.0 ** 100)
    y = oracle.linear(x, p, s)
    np.testing.assert_array_equal(y[0], [2.0 ** -28, -(2.0 ** -27)])


def _moe_edge_layer():
    """Two experts, H = F = 32, one token each (k = 1):
    expert 0: gate row 0 has 6 * 2^127 at element 0, up row 0 has 1.0 there; every down row has
              1.0 at element 0. Token 0, x = 2^-100 at element 0.
    expert 1: gate and up rows 0 have 1.0 at element 0; every down row has 6 * 2^127 at element
              0. Token 1, x = 2^-50 at element 0.
    Everything else is zero."""
    H = F = 32
    gu = np.zeros((2, 2 * F, H), np.uint8)
    gs = np.full((2, 2 * F, 1), 127, np.uint8)
    dn = np.zeros((2, H, F), np.uint8)
    ds = np.full((2, H, 1), 127, np.uint8)
    gu[0, 0, 0], gs[0, 0, 0] = 7, 254
    gu[0, F, 0] = 2
    dn[0, :, 0] = 2
    gu[1, 0, 0] = gu[1, F, 0] = 2
    dn[1, :, 0], ds[1, :, 0] = 7, 254
    gp = np.stack([_pack(g) for g in gu])
    dp = np.stack([_pack(d) for d in dn])
    x = np.zeros((2, H), np.uint16)
    x[0, 0] = _bf16_bits_exact(2.0 ** -100)
    x[1, 0] = _bf16_bits_exact(2.0 ** -50)
    idx = np.array([[0], [1]], np.int32)
    w = np.ones((2, 1), np.float32)
    return x, idx, w, gp, gs, dp, ds


def test_moe_overflowing_weights_bf16_path_and_fp4_path():
    """bf16 path: token 0's gate is +Inf, so h = silu(+Inf) * 2^-100 = +Inf and every output is
    +Inf; token 1's h = bf16(silu(2^-50) * 2^-50) = 2^-101 meets the +Inf down weight: +Inf.
    Activation variant (exact weights): token 0, g = 6 * 2^27 (silu(g) = g in fp64), h = 6 * 2^-73
    (exact in bf16 and MXFP4), output 6 * 2^-73; token 1, h = 2^-101, output 6 * 2^26."""
    x, idx, w, gp, gs, dp, ds = _moe_edge_layer()
    out = oracle.moe_mlp(x, idx, w, gp, gs, dp, ds, E=2)
    assert np.all(out == math.inf)
    out_m = oracle.moe_mlp(x, idx, w, gp, gs, dp, ds, E=2, mx_act=True)
    np.testing.assert_array_equal(out_m[0], np.full(32, 6 * 2.0 ** -73))
    np.testing.assert_array_equal(out_m[1], np.full(32, 6 * 2.0 ** 26))
