"""GPU parity of mxfp4_linear and mxfp4_moe_mlp against the oracle (tolerance bound).

Shapes span several tiles with ragged tails (rows per expert, N not a multiple of the tile, K not
a multiple of the K tile), the decode- and prefill-shaped tile configurations, and the full-size
layers, every token of them against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_weight_quantized_amd import inputs
import mxfp4_weight_quantized_amd as mx
from parity_util import (DEV, bf16_host_bits, check_bf16_output, check_full_layer,
                         check_tolerance, moe_weights, moe_weights_dev, note, to_dev, to_f64)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------------------------ linear
def _linear_case(M, K, N, seed, out_dtype):
    x = inputs.activations(seed, M, K)
    w = inputs.linear_weight_f32(seed, N, K)
    p, s = oracle.quantize(w)
    note("linear M=%d K=%d N=%d %s" % (M, K, N, out_dtype))
    y = mx.mxfp4_linear(to_dev(x), to_dev(p), to_dev(s), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y, oracle.linear(x, p, s)


def test_linear_single_layer_4x256x512():
    """4 x 256 bf16 activations, 512 x 256 weights, fp32 out, seed 0."""
    y, ref = _linear_case(4, 256, 512, 0, torch.float32)
    check_tolerance(to_f64(y), ref, "linear 4x256x512")


@pytest.mark.parametrize("M", [1, 8, 32])
def test_linear_decode_sweep_bf16(M):
    """K = 2880, N = 5760, bf16 out, seed 1."""
    y, ref = _linear_case(M, 2880, 5760, 1, torch.bfloat16)
    y32, _ = _linear_case(M, 2880, 5760, 1, torch.float32)
    check_tolerance(to_f64(y32), ref, "linear M=%d fp32" % M)
    check_bf16_output(bf16_host_bits(y), ref, "linear M=%d" % M, got_f32=to_f64(y32))


@pytest.mark.parametrize("M,K,N", [(1, 32, 16), (17, 96, 200), (5, 64, 48), (100, 2880, 300),
                                   (130, 320, 130), (3, 8192, 64), (257, 2880, 96),
                                   # scale arrays of N*K/32 bytes that are not whole dwords
                                   (3, 32, 17), (100, 96, 33), (70, 160, 7),
                                   # K split over workgroups (decode-sized M): bytewise scales
                                   # with a ragged N, and ragged M over three row tiles
                                   (3, 2880, 17), (33, 2880, 200)])
def test_linear_ragged(M, K, N):
    y, ref = _linear_case(M, K, N, 7 + M, torch.float32)
    check_tolerance(to_f64(y), ref, "linear %dx%dx%d" % (M, K, N))


# ------------------------------------------------------------------------------------ MoE MLP
def _routing(T, E, k, seed):
    r = np.random.default_rng(seed)
    idx = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = r.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    return idx, w


def _run_moe(x, weights_dev, k, out_dtype, wr=None, br=None, idx=None, w=None):
    gp, gs, dp, ds = weights_dev
    out, routing = mx.mxfp4_moe_mlp(
        to_dev(x), gp, gs, dp, ds, k, wr=None if wr is None else to_dev(wr),
        br=None if br is None else to_dev(br), topk_idx=None if idx is None else to_dev(idx),
        topk_w=None if w is None else to_dev(w), out_dtype=out_dtype, return_routing=True)
    torch.cuda.synchronize()
    return out, routing


@pytest.mark.parametrize("T,H,F,E,k", [(1, 64, 64, 1, 1), (37, 256, 192, 8, 2), (7, 96, 320, 4, 4),
                                       (200, 128, 96, 16, 4), (513, 64, 128, 4, 2)])
def test_moe_small_pinned_routing(T, H, F, E, k):
    seed = 60 + T
    x = inputs.activations(seed, T, H)
    wts = moe_weights(seed, E, H, F)
    idx, w = _routing(T, E, k, seed)
    note("moe pinned T=%d H=%d F=%d E=%d k=%d" % (T, H, F, E, k))
    out, _ = _run_moe(x, moe_weights_dev(seed, E, H, F), k, torch.float32, idx=idx, w=w)
    ref = oracle.moe_mlp(x, idx, w, *wts, E=E)
    check_tolerance(to_f64(out), ref, "moe T=%d" % T)


def test_moe_small_internal_routing_bf16():
    T, H, F, E, k, seed = 50, 256, 128, 8, 2, 70
    x = inputs.activations(seed, T, H)
    wr, br = inputs.router(seed, E, H, bias_std=0.5)
    wts = moe_weights(seed, E, H, F)
    note("moe internal routing T=%d" % T)
    out, (lg, idx, w) = _run_moe(x, moe_weights_dev(seed, E, H, F), k, torch.bfloat16, wr=wr, br=br)
    lg, idx, w = lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    oidx, ow = oracle.topk_softmax(lg, k)
    np.testing.assert_array_equal(idx, oidx)
    ref = oracle.moe_mlp(x, idx, w, *wts, E=E)
    check_bf16_output(bf16_host_bits(out), ref, "moe internal bf16")


def test_moe_is_deterministic():
    T, H, F, E, k, seed = 300, 128, 128, 8, 4, 71
    x = inputs.activations(seed, T, H)
    idx, w = _routing(T, E, k, seed)
    wd = moe_weights_dev(seed, E, H, F)
    a, _ = _run_moe(x, wd, k, torch.float32, idx=idx, w=w)
    b, _ = _run_moe(x, wd, k, torch.float32, idx=idx, w=w)
    assert torch.equal(a, b)


def test_moe_bad_routing_index_is_flagged():
    T, H, F, E, k, seed = 4, 64, 64, 4, 2, 72
    x = inputs.activations(seed, T, H)
    idx, w = _routing(T, E, k, seed)
    idx[2, 1] = 7
    gp, gs, dp, ds = moe_weights_dev(seed, E, H, F)
    out = torch.empty((T, H), dtype=torch.float32, device=DEV)
    xd, idxd, wd = to_dev(x), to_dev(idx), to_dev(w)  # held until the call has completed
    assert mx.get_device_error() == 0
    d = mx.make_moe_desc(xd, gp, gs, dp, ds, k, out, topk_idx=idxd, topk_w=wd)
    ws = torch.empty(mx.mxfp4_moe_mlp_workspace(d), dtype=torch.uint8, device=DEV)
    mx._check(mx.lib().mxfp4_moe_mlp(mx.ctypes.byref(d), ws.data_ptr(), ws.numel(),
                                     mx._stream(None)))
    assert mx.workspace_status(ws) == 1
    assert mx.get_device_error() == mx.MX_DEVERR_ROUTING
    good = [0, 1, 3]
    ref = oracle.moe_mlp(x[good], idx[good], w[good], *moe_weights(seed, E, H, F), E=E)
    check_tolerance(to_f64(out)[good], ref, "moe rows without the bad index")


def test_moe_empty_batch():
    """T = 0: nothing to route or compute; the call succeeds and the output is empty."""
    H, F, E, k, seed = 64, 64, 4, 2, 73
    wr, _ = inputs.router(seed, E, H, 0.0)
    x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    note("moe empty batch")
    out = mx.mxfp4_moe_mlp(x, *moe_weights_dev(seed, E, H, F), k, wr=to_dev(wr),
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, H)


@pytest.mark.parametrize("T", [16, 64])
def test_moe_max_experts_and_topk(T):
    """E = MX_MAX_EXPERTS (256) and k = MX_MAX_TOPK (8), internal routing: four experts per lane
    in the selection, all 256 groups of the permutation (T = 16: selection inside the
    permutation launch; T = 64: its own launch)."""
    H, F, E, k, seed = 128, 64, 256, 8, 75
    x = inputs.activations(seed, T, H)
    wr, br = inputs.router(seed, E, H, bias_std=0.5)
    wts = moe_weights(seed, E, H, F)
    note("moe max experts T=%d E=%d k=%d" % (T, E, k))
    out, (lg, idx, w) = _run_moe(x, moe_weights_dev(seed, E, H, F), k, torch.float32, wr=wr, br=br)
    lg, idx, w = lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    oidx, ow = oracle.topk_softmax(lg, k)
    np.testing.assert_array_equal(idx, oidx)
    np.testing.assert_allclose(w, ow, rtol=2e-6, atol=1e-7)
    ref = oracle.moe_mlp(x, idx, w, *wts, E=E)
    check_tolerance(to_f64(out), ref, "moe E=256 k=8 T=%d" % T)


# ----------------------------------------------------------------------------- full-size layers
FULL_SHAPES = [inputs.MOE_20B_DECODE, inputs.MOE_20B_PREFILL, *inputs.MOE_120B.values()]


@pytest.mark.parametrize("shape", FULL_SHAPES, ids=[s.name for s in FULL_SHAPES])
def test_moe_full_layer_row_major(shape):
    """Every token of the 20B-shaped (T = 64; T = 8192 with the skewed router) and 120B-shaped
    (T = 1, 256, 4096) layers, internal routing, fp32 and bf16 outputs, against one oracle run
    under the oracle's own routing."""
    check_full_layer(shape, flags=0, tiled=False)
