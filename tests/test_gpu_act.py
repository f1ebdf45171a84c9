"""GPU: the parameterised expert activation (biases, clamp, sigmoid scale, up shift, interleaved
gate/up rows) against the oracle's, and the de-interleaving tiled layout.

Interleaved weights are made from the seeded halves-order weights by interleaving their rows on
the host; the GPU tiles them with MX_TILE_DEINTERLEAVE (which must equal tiling the halves-order
weights byte for byte) and reads the gate_up bias in the interleaved order."""
import functools

import numpy as np
import pytest
import torch

import oracle
from mxfp4_weight_quantized_amd import inputs
import mxfp4_weight_quantized_amd as mx
from parity_util import (FRAGILE_C, bf16_host_bits, check_bf16_output, check_tolerance,
                         layer_weights, layer_weights_dev, moe_weights, moe_weights_dev, note,
                         oracle_layer, routing_parity, tiled_dev, to_dev, to_f64)

pytestmark = pytest.mark.gpu

MX = mx.MX_ACT_MXFP4
TILED = mx.MX_WEIGHTS_TILED
RELEASED = dict(alpha=1.702, limit=7.0, up_shift=1.0)


def _interleave(a):
    """[E, 2F, ...] rows [0, F) gate, [F, 2F) up -> row 2i gate i, row 2i + 1 up i."""
    F = a.shape[1] // 2
    out = np.empty_like(a)
    out[:, 0::2], out[:, 1::2] = a[:, :F], a[:, F:]
    return out


def _np_tile_deinterleave(packed, scales):
    G, R, Kh = packed.shape
    nb = scales.shape[2]
    p = np.concatenate([packed[:, 0::2], packed[:, 1::2]], axis=1)
    s = np.concatenate([scales[:, 0::2], scales[:, 1::2]], axis=1)
    pt = p.reshape(G, R // 16, 16, nb, 16).transpose(0, 1, 3, 2, 4)
    st = s.transpose(0, 2, 1)
    return np.ascontiguousarray(pt).reshape(G, R, Kh), np.ascontiguousarray(st).reshape(G, R, nb)


@pytest.mark.parametrize("G,R,K", [(1, 32, 32), (3, 64, 96), (2, 5760, 2880)])
def test_tile_weights_deinterleave_is_the_documented_permutation(G, R, K):
    r = np.random.default_rng(G + R + K)
    packed = r.integers(0, 256, size=(G, R, K // 2), dtype=np.uint8)
    scales = r.integers(0, 256, size=(G, R, K // 32), dtype=np.uint8)
    note("tile_weights deinterleave G=%d R=%d K=%d" % (G, R, K))
    pt, st = mx.mxfp4_tile_weights(to_dev(packed), to_dev(scales), deinterleave=True)
    torch.cuda.synchronize()
    ept, est = _np_tile_deinterleave(packed, scales)
    np.testing.assert_array_equal(pt.cpu().numpy(), ept)
    np.testing.assert_array_equal(st.cpu().numpy(), est)


def _routing(T, E, k, seed):
    r = np.random.default_rng(seed)
    idx = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = r.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    return idx, w


def _biases(seed, E, H, F, std):
    r = np.random.default_rng(seed)
    return (r.normal(0, std, (E, 2 * F)).astype(np.float32),
            r.normal(0, std, (E, H)).astype(np.float32))


# decode- and prefill-shaped tiles; biases of std 4 push many gate/up values past the limit of 7
@pytest.mark.parametrize("T,H,F,E,k", [(37, 256, 192, 8, 2), (7, 96, 320, 4, 4),
                                       (600, 256, 320, 2, 1), (300, 128, 96, 4, 4)])
@pytest.mark.parametrize("flags", [0, MX])
@pytest.mark.parametrize("interleaved", [False, True])
def test_moe_act_small_pinned_routing(T, H, F, E, k, flags, interleaved):
    seed = 700 + T
    x = inputs.activations(seed, T, H)
    gp, gs, dp, ds = moe_weights(seed, E, H, F)
    gb, db = _biases(seed, E, H, F, 4.0)
    idx, w = _routing(T, E, k, seed)
    if interleaved:
        gp, gs, gb = _interleave(gp), _interleave(gs), _interleave(gb)
    o_act = dict(RELEASED, interleaved=interleaved, gu_bias=gb, dn_bias=db)
    g_act = dict(RELEASED, interleaved=interleaved, gu_bias=to_dev(gb), dn_bias=to_dev(db))
    gpt, gst = mx.mxfp4_tile_weights(to_dev(gp), to_dev(gs), deinterleave=interleaved)
    dpt, dst = mx.mxfp4_tile_weights(to_dev(dp), to_dev(ds))
    note("moe act T=%d H=%d F=%d E=%d k=%d flags=%d interleaved=%d" % (T, H, F, E, k, flags,
                                                                        interleaved))
    out = mx.mxfp4_moe_mlp(to_dev(x), gpt, gst, dpt, dst, k, topk_idx=to_dev(idx),
                           topk_w=to_dev(w), out_dtype=torch.float32, flags=flags | TILED,
                           act=g_act)
    torch.cuda.synchronize()
    if flags & MX:
        ref, _, slack = oracle.moe_mlp(x, idx, w, gp, gs, dp, ds, E=E, mx_act=True,
                                       fragile_c=FRAGILE_C, act=o_act)
    else:
        ref, slack = oracle.moe_mlp(x, idx, w, gp, gs, dp, ds, E=E, act=o_act), None
    check_tolerance(to_f64(out), ref, "moe act T=%d" % T, slack=slack)
    # the clamp is reached in these cases (biases alone put ~8 % of the values past the limit)
    assert (np.abs(gb) > RELEASED["limit"]).mean() > 0.02
    if not interleaved and not flags:  # row-major weights: the same output as the tiled layout
        rm = mx.mxfp4_moe_mlp(to_dev(x), *moe_weights_dev(seed, E, H, F), k, topk_idx=to_dev(idx),
                              topk_w=to_dev(w), out_dtype=torch.float32, act=g_act)
        torch.cuda.synchronize()
        assert torch.equal(rm, out)


@pytest.mark.parametrize("flags", [0, MX])
def test_moe_act_zero_parameters_are_the_plain_path(flags):
    """The expert activation fields all zero, and a descriptor that ends before them, give the
    plain SwiGLU bit for bit."""
    T, H, F, E, k, seed = 40, 128, 96, 4, 2, 760
    x = to_dev(inputs.activations(seed, T, H))
    wd = moe_weights_dev(seed, E, H, F)
    idx, w = _routing(T, E, k, seed)
    kw = dict(topk_idx=to_dev(idx), topk_w=to_dev(w), out_dtype=torch.float32, flags=flags)
    plain = mx.mxfp4_moe_mlp(x, *wd, k, **kw)
    zero = mx.mxfp4_moe_mlp(x, *wd, k, act=dict(alpha=0.0, limit=0.0, up_shift=0.0), **kw)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    d = mx.make_moe_desc(x, *wd, k, out, topk_idx=kw["topk_idx"], topk_w=kw["topk_w"],
                         flags=flags)
    d.struct_size = mx.MoeDesc.act_flags.offset
    ws = torch.empty(mx.mxfp4_moe_mlp_workspace(d), dtype=torch.uint8, device="cuda")
    mx._check(mx.lib().mxfp4_moe_mlp(mx.ctypes.byref(d), ws.data_ptr(), ws.numel(),
                                     mx._stream(None)))
    torch.cuda.synchronize()
    assert torch.equal(plain, zero) and torch.equal(plain, out)


# ------------------------------------------------------------------------- full-size layers
@functools.lru_cache(maxsize=4)
def _act_layer(shape):
    """Interleaved gate_up weights and biases for a full-size layer (host), and the released
    activation parameters for the oracle and the GPU."""
    gp, gs, dp, ds = layer_weights(shape.seed, shape.E, shape.H, shape.F)
    gb, db = _biases(shape.seed + 11, shape.E, shape.H, shape.F, 0.1)
    return _interleave(gp), _interleave(gs), dp, ds, _interleave(gb), db


@functools.lru_cache(maxsize=4)
def _act_oracle(shape, mx_act):
    x, _, _, _, idx, w = oracle_layer(shape)
    gp, gs, dp, ds, gb, db = _act_layer(shape)
    act = dict(RELEASED, interleaved=True, gu_bias=gb, dn_bias=db)
    note("oracle: %s with the released activation%s" % (shape.name, " (FP4 act)" if mx_act else ""))
    if mx_act:
        out, _, slack = oracle.moe_mlp(x, idx, w, gp, gs, dp, ds, E=shape.E, mx_act=True,
                                       fragile_c=FRAGILE_C, act=act)
        return out, slack
    return oracle.moe_mlp(x, idx, w, gp, gs, dp, ds, E=shape.E, act=act), None


@pytest.mark.parametrize("shape,flags", [(inputs.MOE_20B_DECODE, 0), (inputs.MOE_20B_DECODE, MX),
                                         (inputs.MOE_20B_PREFILL, 0), (inputs.MOE_120B[256], 0)],
                         ids=["20b-decode", "20b-decode-fp4act", "20b-prefill", "120b-T256"])
def test_moe_act_full_layer(shape, flags):
    """Every token of a full-size layer with the released model's activation (alpha 1.702,
    limit 7, up shift 1, biases) and interleaved gate/up rows, internal routing, fp32 and bf16
    outputs, against the oracle."""
    s = shape
    gp, gs, dp, ds, gb, db = _act_layer(s)
    gpt, gst = mx.mxfp4_tile_weights(to_dev(gp), to_dev(gs), deinterleave=True)
    # de-interleaving while tiling gives the halves-order layer's tiled weights byte for byte
    hp, hs, _, _ = tiled_dev(layer_weights_dev(s.seed, s.E, s.H, s.F))
    assert torch.equal(gpt, hp) and torch.equal(gst, hs)
    dpt, dst = mx.mxfp4_tile_weights(to_dev(dp), to_dev(ds))
    x, wr, br, _, _, _ = oracle_layer(s)
    act = dict(RELEASED, interleaved=True, gu_bias=to_dev(gb), dn_bias=to_dev(db))
    ref, slack = _act_oracle(s, bool(flags & MX))
    got32 = None
    for out_dtype in (torch.float32, torch.bfloat16):
        note("moe act full %s flags=%d %s" % (s.name, flags, out_dtype))
        out, (lg, idx, w) = mx.mxfp4_moe_mlp(
            to_dev(x), gpt, gst, dpt, dst, s.k, wr=to_dev(wr), br=None if br is None else to_dev(br),
            out_dtype=out_dtype, flags=flags | TILED, return_routing=True, act=act)
        torch.cuda.synchronize()
        ties, _, _ = routing_parity(s, lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy())
        assert len(ties) == 0, "near-tie routing: compare those tokens separately"
        what = "%s act flags=%d %s" % (s.name, flags, out_dtype)
        if out_dtype == torch.float32:
            got32 = to_f64(out)
            check_tolerance(got32, ref, what, slack=slack)
        else:
            check_bf16_output(bf16_host_bits(out), ref, what, slack=slack, got_f32=got32)
