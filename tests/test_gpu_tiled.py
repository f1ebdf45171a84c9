"""GPU: the tiled weight layout (mxfp4_tile_weights) and the grouped GEMMs that read it.

The layout is a byte permutation; it is checked bit-exactly against the same permutation written
with numpy reshapes. On tiled weights the MoE MLP performs the same arithmetic in the same order
as on row-major weights (only the addresses the weight stages come from differ), so its output
must equal the row-major output bit for bit, for the bf16 path and the activation variant, on the
decode-shaped and the prefill-shaped tile paths. The 20B and 120B shapes are also checked
against the oracle directly."""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_weight_quantized_amd import inputs
import mxfp4_weight_quantized_amd as mx
from parity_util import (FRAGILE_C, check_full_layer, check_tolerance, layer_weights_dev,
                         moe_weights, moe_weights_dev, note, tiled_dev, to_dev, to_f64)

pytestmark = pytest.mark.gpu

TILED = mx.MX_WEIGHTS_TILED


def _np_tile(packed, scales):
    """codes [G][R][K/2] -> [G][R/16][K/32][16 rows][16 bytes]; scales [G][R][K/32] -> [G][K/32][R]
    (returned with the input shapes, as the binding does)."""
    G, R, Kh = packed.shape
    nb = scales.shape[2]
    pt = packed.reshape(G, R // 16, 16, nb, 16).transpose(0, 1, 3, 2, 4)
    st = scales.transpose(0, 2, 1)
    return np.ascontiguousarray(pt).reshape(G, R, Kh), np.ascontiguousarray(st).reshape(G, R, nb)


@pytest.mark.parametrize("G,R,K", [(1, 16, 32), (3, 32, 64), (4, 192, 96), (2, 256, 2880),
                                   (5, 48, 320)])
def test_tile_weights_is_the_documented_permutation(G, R, K):
    r = np.random.default_rng(G * 1000 + R + K)
    packed = r.integers(0, 256, size=(G, R, K // 2), dtype=np.uint8)
    scales = r.integers(0, 256, size=(G, R, K // 32), dtype=np.uint8)
    note("tile_weights G=%d R=%d K=%d" % (G, R, K))
    pt, st = mx.mxfp4_tile_weights(to_dev(packed), to_dev(scales))
    torch.cuda.synchronize()
    ept, est = _np_tile(packed, scales)
    np.testing.assert_array_equal(pt.cpu().numpy(), ept)
    np.testing.assert_array_equal(st.cpu().numpy(), est)


def _routing(T, E, k, seed):
    r = np.random.default_rng(seed)
    idx = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = r.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    return idx, w


# decode-shaped tiles (T*k < 64E) and prefill-shaped tiles (T*k >= 64E), F below one tile too
@pytest.mark.parametrize("T,H,F,E,k", [(1, 64, 64, 1, 1), (37, 256, 192, 8, 2), (7, 96, 320, 4, 4),
                                       (513, 64, 128, 4, 2), (300, 128, 96, 4, 4),
                                       (600, 256, 320, 2, 1)])
@pytest.mark.parametrize("flags", [0, mx.MX_ACT_MXFP4])
def test_moe_tiled_equals_row_major(T, H, F, E, k, flags):
    seed = 300 + T
    x = to_dev(inputs.activations(seed, T, H))
    wd = moe_weights_dev(seed, E, H, F)
    idx, w = _routing(T, E, k, seed)
    idx_d, w_d = to_dev(idx), to_dev(w)
    note("moe tiled vs row-major T=%d H=%d F=%d E=%d k=%d flags=%d" % (T, H, F, E, k, flags))
    a = mx.mxfp4_moe_mlp(x, *wd, k, topk_idx=idx_d, topk_w=w_d, out_dtype=torch.float32,
                         flags=flags)
    b = mx.mxfp4_moe_mlp(x, *tiled_dev(wd), k, topk_idx=idx_d, topk_w=w_d, out_dtype=torch.float32,
                         flags=flags | TILED)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("flags", [0, mx.MX_ACT_MXFP4])
def test_moe_tiled_equals_row_major_20b_prefill(flags):
    s = inputs.MOE_20B_PREFILL
    x = to_dev(inputs.activations(s.seed, s.T, s.H))
    wr, br = inputs.router(s.seed, s.E, s.H, s.bias_std)
    wd = layer_weights_dev(s.seed, s.E, s.H, s.F)
    note("moe tiled vs row-major %s flags=%d" % (s.name, flags))
    kw = dict(wr=to_dev(wr), br=to_dev(br) if s.bias_std else None, out_dtype=torch.bfloat16)
    a = mx.mxfp4_moe_mlp(x, *wd, s.k, flags=flags, **kw)
    b = mx.mxfp4_moe_mlp(x, *tiled_dev(wd), s.k, flags=flags | TILED, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# H = F = MX_MAX_MOE_DIM (3072): decode tiles hold exactly 96 blocks of resident scales per row;
# prefill tiles end K with a full stage. Internal routing, row-major and tiled weights.
@pytest.mark.parametrize("T,E,k,tiled", [(9, 4, 2, False), (9, 4, 2, True), (200, 2, 1, True)])
def test_moe_max_dims(T, E, k, tiled):
    H = F = 3072
    seed = 76 + T
    x = inputs.activations(seed, T, H)
    wr, br = inputs.router(seed, E, H, 0.5)
    wts = moe_weights(seed, E, H, F)
    wd = moe_weights_dev(seed, E, H, F)
    note("moe max dims T=%d H=F=%d E=%d k=%d tiled=%d" % (T, H, E, k, tiled))
    out, (lg, idx, w) = mx.mxfp4_moe_mlp(
        to_dev(x), *(tiled_dev(wd) if tiled else wd), k, wr=to_dev(wr), br=to_dev(br),
        out_dtype=torch.float32, flags=TILED if tiled else 0, return_routing=True)
    torch.cuda.synchronize()
    lg, idx, w = lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    oidx, ow = oracle.topk_softmax(lg, k)
    np.testing.assert_array_equal(idx, oidx)
    ref = oracle.moe_mlp(x, idx, w, *wts, E=E)
    check_tolerance(to_f64(out), ref, "moe H=F=3072 T=%d" % T)


# Few pairs and a long K (the few-tile GEMM configurations over all their stages), for the bf16
# path and the activation variant: tiled equals row-major bit for bit, and both match the oracle.
@pytest.mark.parametrize("T,H,F,E,k", [(2, 2880, 2880, 8, 2), (3, 2880, 1440, 16, 4)])
@pytest.mark.parametrize("flags", [0, mx.MX_ACT_MXFP4])
def test_moe_few_pairs_long_k(T, H, F, E, k, flags):
    seed = 90 + T
    x = inputs.activations(seed, T, H)
    wts = moe_weights(seed, E, H, F)
    wd = moe_weights_dev(seed, E, H, F)
    idx, w = _routing(T, E, k, seed)
    idx_d, w_d = to_dev(idx), to_dev(w)
    note("moe few pairs T=%d H=%d F=%d E=%d k=%d flags=%d" % (T, H, F, E, k, flags))
    a = mx.mxfp4_moe_mlp(to_dev(x), *wd, k, topk_idx=idx_d, topk_w=w_d, out_dtype=torch.float32,
                         flags=flags)
    b = mx.mxfp4_moe_mlp(to_dev(x), *tiled_dev(wd), k, topk_idx=idx_d, topk_w=w_d,
                         out_dtype=torch.float32, flags=flags | TILED)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    if flags & mx.MX_ACT_MXFP4:
        ref, _, slack = oracle.moe_mlp(x, idx, w, *wts, E=E, mx_act=True, fragile_c=FRAGILE_C)
        check_tolerance(to_f64(b), ref, "moe mx-act few pairs T=%d" % T, slack=slack)
    else:
        check_tolerance(to_f64(b), oracle.moe_mlp(x, idx, w, *wts, E=E), "moe few pairs T=%d" % T)


FULL_SHAPES = [inputs.MOE_20B_DECODE, inputs.MOE_20B_PREFILL, *inputs.MOE_120B.values()]


@pytest.mark.parametrize("shape", FULL_SHAPES, ids=[s.name for s in FULL_SHAPES])
def test_moe_full_layer_tiled(shape):
    """The benchmarked weight layout: every token of the full-size layers against the oracle,
    fp32 and bf16 outputs."""
    check_full_layer(shape, flags=0, tiled=True)
