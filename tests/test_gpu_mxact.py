"""GPU parity of the activation variant (MX_ACT_MXFP4): activations quantized to MXFP4 on the
fly and every product run on the scaled FP4 MFMA, against the oracle's activation variant.

The quantization of x is a decision on bf16 inputs both sides share, so it is exact. The one of
h follows an fp32 (GPU) or fp64 (oracle) gate/up sum; the oracle flags the h decisions an fp32
implementation may take the other way and the per-element bound is widened by the slack they
allow (see test_oracle_fragile.py for the pins of that aid)."""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_weight_quantized_amd import inputs
import mxfp4_weight_quantized_amd as mx
from parity_util import (DEV, FRAGILE_C, bf16_host_bits, check_bf16_output, check_full_layer,
                         check_tolerance, moe_weights, moe_weights_dev, note, to_dev, to_f64)

pytestmark = pytest.mark.gpu

MX = mx.MX_ACT_MXFP4


# ------------------------------------------------------------------------------------ linear
def _linear_case(M, K, N, seed, out_dtype):
    x = inputs.activations(seed, M, K)
    w = inputs.linear_weight_f32(seed, N, K)
    p, s = oracle.quantize(w)
    note("linear mx-act M=%d K=%d N=%d %s" % (M, K, N, out_dtype))
    y = mx.mxfp4_linear(to_dev(x), to_dev(p), to_dev(s), out_dtype=out_dtype, flags=MX)
    torch.cuda.synchronize()
    return y, oracle.linear(x, p, s, mx_act=True)


@pytest.mark.parametrize("M,N", [(1, 16), (37, 200), (130, 96), (5, 17), (90, 7)])
def test_linear_mxact_single_block_is_exact(M, N):
    """K = 32: one block per dot product, so every partial sum of the FP4 x FP4 products (codes
    with two significant bits, one shared pair of power-of-two scales) is exact in fp32 and the
    GPU result must equal the oracle's exactly."""
    y, ref = _linear_case(M, 32, N, 90 + M, torch.float32)
    np.testing.assert_array_equal(to_f64(y), ref)


@pytest.mark.parametrize("M", [1, 8, 32])
def test_linear_mxact_decode_sweep(M):
    """K = 2880, N = 5760."""
    y, ref = _linear_case(M, 2880, 5760, 1, torch.float32)
    check_tolerance(to_f64(y), ref, "linear mx-act M=%d" % M)
    yb, _ = _linear_case(M, 2880, 5760, 1, torch.bfloat16)
    check_bf16_output(bf16_host_bits(yb), ref, "linear mx-act M=%d bf16" % M, got_f32=to_f64(y))


@pytest.mark.parametrize("M,K,N", [(17, 96, 200), (5, 64, 48), (100, 2880, 300), (130, 320, 130),
                                   (3, 8192, 64), (257, 2880, 96), (9, 96, 33), (100, 160, 7)])
def test_linear_mxact_ragged(M, K, N):
    y, ref = _linear_case(M, K, N, 7 + M, torch.float32)
    check_tolerance(to_f64(y), ref, "linear mx-act %dx%dx%d" % (M, K, N))


# ------------------------------------------------------------------------------------ MoE MLP
def _routing(T, E, k, seed):
    r = np.random.default_rng(seed)
    idx = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = r.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    return idx, w


def _run(x, wdev, k, out_dtype, wr=None, br=None, idx=None, w=None):
    gp, gs, dp, ds = wdev
    out, routing = mx.mxfp4_moe_mlp(
        to_dev(x), gp, gs, dp, ds, k, wr=None if wr is None else to_dev(wr),
        br=None if br is None else to_dev(br), topk_idx=None if idx is None else to_dev(idx),
        topk_w=None if w is None else to_dev(w), out_dtype=out_dtype, flags=MX,
        return_routing=True)
    torch.cuda.synchronize()
    return out, routing


@pytest.mark.parametrize("T,H,F,E,k", [(1, 64, 64, 1, 1), (37, 256, 192, 8, 2), (7, 96, 320, 4, 4),
                                       (200, 128, 96, 16, 4), (513, 64, 128, 4, 2)])
def test_moe_mxact_small_pinned_routing(T, H, F, E, k):
    seed = 160 + T
    x = inputs.activations(seed, T, H)
    wts = moe_weights(seed, E, H, F)
    idx, w = _routing(T, E, k, seed)
    note("moe mx-act pinned T=%d H=%d F=%d E=%d k=%d" % (T, H, F, E, k))
    out, _ = _run(x, moe_weights_dev(seed, E, H, F), k, torch.float32, idx=idx, w=w)
    ref, _, slack = oracle.moe_mlp(x, idx, w, *wts, E=E, mx_act=True, fragile_c=FRAGILE_C)
    check_tolerance(to_f64(out), ref, "moe mx-act T=%d" % T, slack=slack)


# Routing indices outside [0, E) leave their pairs out (their inv is -1) and set the device error
# word. Decode-shaped (16-row tiles: x's codes in token order, gathered) and prefill-shaped
# (128-row tiles: x's and h's codes copied into pair order, tiled by 16 rows; P = 1026 leaves a
# partial last group of 16): the reference is the oracle with those pairs' weights at zero.
@pytest.mark.parametrize("T,H,F,E,k", [(40, 128, 96, 8, 2), (513, 64, 128, 4, 2)])
def test_moe_mxact_skips_out_of_range_indices(T, H, F, E, k):
    seed = 180 + T
    x = inputs.activations(seed, T, H)
    wts = moe_weights(seed, E, H, F)
    idx, w = _routing(T, E, k, seed)
    idx[3, 1], idx[7, 0], idx[T - 1, 1] = -1, E, E + 5
    ref_idx, ref_w = idx.copy(), w.copy()
    bad = (idx < 0) | (idx >= E)
    ref_idx[bad], ref_w[bad] = 0, 0.0
    mx.get_device_error()  # clear
    note("moe mx-act out-of-range indices T=%d E=%d" % (T, E))
    out, _ = _run(x, moe_weights_dev(seed, E, H, F), k, torch.float32, idx=idx, w=w)
    assert mx.get_device_error() == mx.MX_DEVERR_ROUTING
    ref, _, slack = oracle.moe_mlp(x, ref_idx, ref_w, *wts, E=E, mx_act=True, fragile_c=FRAGILE_C)
    check_tolerance(to_f64(out), ref, "moe mx-act skipped pairs T=%d" % T, slack=slack)


def test_moe_mxact_is_deterministic():
    T, H, F, E, k, seed = 300, 128, 128, 8, 4, 171
    x = inputs.activations(seed, T, H)
    idx, w = _routing(T, E, k, seed)
    wd = moe_weights_dev(seed, E, H, F)
    a, _ = _run(x, wd, k, torch.float32, idx=idx, w=w)
    b, _ = _run(x, wd, k, torch.float32, idx=idx, w=w)
    assert torch.equal(a, b)


FULL_SHAPES = [inputs.MOE_20B_DECODE, inputs.MOE_20B_PREFILL, *inputs.MOE_120B.values()]


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("shape", FULL_SHAPES, ids=[s.name for s in FULL_SHAPES])
def test_moe_mxact_full_layer(shape, tiled):
    """Every token of the full-size layers with activations quantized on the fly, fp32 and bf16
    outputs, against one oracle run of the activation variant (with its fragile-decision
    slack)."""
    check_full_layer(shape, flags=MX, tiled=tiled)
