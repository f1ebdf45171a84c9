"""GPU: the MoE MLP as one launch (MX_SINGLE_LAUNCH) against the oracle, and against the same call
made of one launch per step.

With the caller's routing both forms run the same decode tiles with the same operations in the
same order, so their outputs agree bit for bit (fp32 and bf16, plain and expert-activation
variants, out-of-range routing indices included). With internal routing the router's logits are
summed over a different split of H, so the routing is checked like the router's own (logits by
tolerance against the oracle, indices exact given the logits) and every output element against
the oracle. Consecutive calls in one process also check that each call leaves the launch's
counters at zero for the next one."""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_weight_quantized_amd import inputs
import mxfp4_weight_quantized_amd as mx
from parity_util import (check_full_layer, check_tolerance, moe_weights, note, tiled_dev, to_dev,
                         to_f64)

pytestmark = pytest.mark.gpu

S = mx.MX_SINGLE_LAUNCH
TILED = mx.MX_WEIGHTS_TILED


def _routing(T, E, k, seed):
    r = np.random.default_rng(seed)
    idx = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = r.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    return idx, w


def _both(x, wd, k, idx, w, flags, out_dtype, act=None):
    kw = dict(topk_idx=idx, topk_w=w, out_dtype=out_dtype, act=act)
    split = mx.mxfp4_moe_mlp(x, *wd, k, flags=flags, **kw)
    single = mx.mxfp4_moe_mlp(x, *wd, k, flags=flags | S, **kw)
    torch.cuda.synchronize()
    return split, single


# decode-shaped problems (T*k < 64 E: decode tiles in both forms), few-expert (T = 1) included,
# and the largest batches the single launch takes (T*k = 2048: 128 token tiles, and with E = 256
# the longest tile list, 384 row tiles)
CASES = [(1, 2880, 2880, 128, 4), (5, 256, 192, 8, 2), (37, 256, 320, 16, 4),
         (64, 2880, 2880, 32, 4), (130, 128, 96, 8, 1), (17, 96, 64, 256, 8),
         (2048, 128, 96, 256, 1), (256, 128, 64, 256, 8)]


@pytest.mark.parametrize("T,H,F,E,k", CASES)
@pytest.mark.parametrize("tiled", [False, True])
def test_single_equals_split_launches(T, H, F, E, k, tiled):
    seed = 900 + T + E
    x = to_dev(inputs.activations(seed, T, H))
    gp, gs, dp, ds = moe_weights(seed, E, H, F)
    wd = tuple(to_dev(a) for a in (gp, gs, dp, ds))
    if tiled:
        wd = tiled_dev(wd)
    idx, w = _routing(T, E, k, seed)
    fl = TILED if tiled else 0
    for out_dtype in (torch.float32, torch.bfloat16):
        note("single vs split T=%d H=%d F=%d E=%d k=%d tiled=%d %s" % (T, H, F, E, k, tiled, out_dtype))
        split, single = _both(x, wd, k, to_dev(idx), to_dev(w), fl, out_dtype)
        assert torch.equal(split, single)
        if out_dtype == torch.float32 and T * H * F <= 256 * 256 * 320:
            ref = oracle.moe_mlp(inputs.activations(seed, T, H), idx, w, gp, gs, dp, ds, E=E)
            check_tolerance(to_f64(single), ref, "single T=%d" % T)
    assert mx.get_device_error() == 0


def test_single_expert_activation_equals_split():
    """Biases, clamp, sigmoid scale and up shift, interleaved gate/up rows."""
    T, H, F, E, k, seed = 48, 256, 192, 8, 2, 950
    r = np.random.default_rng(seed)
    x = to_dev(inputs.activations(seed, T, H))
    gp, gs, dp, ds = moe_weights(seed, E, H, F)
    inter = lambda a: np.stack([a[:, :F], a[:, F:]], axis=2).reshape(a.shape)  # rows 2i, 2i + 1
    gb = r.normal(0, 4.0, (E, 2 * F)).astype(np.float32)
    db = r.normal(0, 4.0, (E, H)).astype(np.float32)
    gpt, gst = mx.mxfp4_tile_weights(to_dev(inter(gp)), to_dev(inter(gs)), deinterleave=True)
    dpt, dst = mx.mxfp4_tile_weights(to_dev(dp), to_dev(ds))
    act = dict(alpha=1.702, limit=7.0, up_shift=1.0, interleaved=True, gu_bias=to_dev(inter(gb)),
               dn_bias=to_dev(db))
    idx, w = _routing(T, E, k, seed)
    for out_dtype in (torch.float32, torch.bfloat16):
        note("single vs split, expert activation, %s" % out_dtype)
        split, single = _both(x, (gpt, gst, dpt, dst), k, to_dev(idx), to_dev(w), TILED, out_dtype,
                              act=act)
        assert torch.equal(split, single)


def test_single_skips_out_of_range_indices():
    T, H, F, E, k, seed = 20, 128, 96, 8, 2, 960
    x = to_dev(inputs.activations(seed, T, H))
    wd = tuple(to_dev(a) for a in moe_weights(seed, E, H, F))
    idx, w = _routing(T, E, k, seed)
    idx[3, 1], idx[7, 0], idx[11, 1] = -1, E, E + 5
    mx.get_device_error()  # clear
    note("single with out-of-range indices")
    split, single = _both(x, wd, k, to_dev(idx), to_dev(w), 0, torch.float32)
    assert torch.equal(split, single)
    assert mx.get_device_error() == mx.MX_DEVERR_ROUTING
    # every index out of range: no pair reaches a GEMM and the output is zero
    bad = np.full_like(idx, E + 1)
    note("single with every index out of range")
    split, single = _both(x, wd, k, to_dev(bad), to_dev(w), 0, torch.float32)
    assert torch.equal(split, single) and not torch.any(single)
    assert mx.get_device_error() == mx.MX_DEVERR_ROUTING


def test_single_back_to_back_problems():
    """Different problem sizes one after another without synchronizing in between, then the
    first again: each call must leave the launch's counters at zero for the next."""
    runs = []
    for (T, H, F, E, k) in [(33, 256, 192, 16, 4), (3, 128, 64, 4, 1), (33, 256, 192, 16, 4)]:
        seed = 970 + T
        x = to_dev(inputs.activations(seed, T, H))
        wd = tuple(to_dev(a) for a in moe_weights(seed, E, H, F))
        idx, w = _routing(T, E, k, seed)
        note("single back to back T=%d E=%d" % (T, E))
        runs.append(mx.mxfp4_moe_mlp(x, *wd, k, topk_idx=to_dev(idx), topk_w=to_dev(w),
                                     out_dtype=torch.float32, flags=S))
    torch.cuda.synchronize()
    assert torch.equal(runs[0], runs[2])
    assert mx.get_device_error() == 0


# (and a small layer at the launch's limit of 2048 pairs, internal routing over 32 token tiles)
LIMIT = inputs.MoEShape("moe-limit-T512", T=512, H=256, F=256, E=32, k=4, seed=981)


@pytest.mark.parametrize("shape,tiled", [(inputs.MOE_20B_DECODE, True), (inputs.MOE_20B_DECODE, False),
                                         (inputs.MOE_120B[1], True), (inputs.MOE_120B[256], True),
                                         (LIMIT, True)],
                         ids=["20b-decode-tiled", "20b-decode-rowmajor", "120b-T1", "120b-T256",
                              "limit-T512"])
def test_single_full_layer(shape, tiled):
    """Every token of a full-size layer with internal routing, fp32 and bf16 outputs, against
    the oracle."""
    check_full_layer(shape, S, tiled=tiled)
    assert mx.get_device_error() == 0


def test_single_through_the_allocation_free_entry_point():
    """MX_SINGLE_LAUNCH with the library's own workspace: the same output as with a caller
    workspace, twice in a row (the second call smaller)."""
    for (T, H, F, E, k) in [(40, 256, 192, 16, 4), (9, 128, 96, 8, 2)]:
        seed = 990 + T
        x = to_dev(inputs.activations(seed, T, H))
        wd = tiled_dev(tuple(to_dev(a) for a in moe_weights(seed, E, H, F)))
        wr, _ = inputs.router(seed, E, H, 0.0)
        kw = dict(wr=to_dev(wr), out_dtype=torch.float32, flags=S | TILED)
        ref = mx.mxfp4_moe_mlp(x, *wd, k, **kw)
        out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        d = mx.make_moe_desc(x, *wd, k, out, wr=kw["wr"], flags=S | TILED)
        note("single, allocation-free entry point, T=%d" % T)
        mx.mxfp4_moe_mlp_noalloc(d)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    assert mx.get_device_error() == 0
