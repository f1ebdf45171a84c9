"""GPU parity of moe_route_topk and moe_permute.

Logits are compared with the oracle's by tolerance (fp32 sums in a different order); the top-k
indices must equal the oracle's top-k taken on the GPU's own logits, bit for bit, and the
permutation must equal the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_weight_quantized_amd import inputs
import mxfp4_weight_quantized_amd as mx
from parity_util import DEV, moe_weights_dev, note, to_dev

pytestmark = pytest.mark.gpu


def _route(T, H, E, k, seed, bias_std=0.0, wr=None):
    x = inputs.activations(seed, T, H)
    wr_, br = inputs.router(seed, E, H, bias_std)
    if wr is not None:
        wr_ = wr
    note("route T=%d H=%d E=%d k=%d" % (T, H, E, k))
    lg, idx, w = mx.moe_route_topk(to_dev(x), to_dev(wr_), to_dev(br) if bias_std else None, k)
    torch.cuda.synchronize()
    return x, wr_, (br if bias_std else None), lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("T,H,E,k,bias", [(1, 2880, 128, 4, 0.0), (5, 64, 8, 1, 0.0),
                                          (37, 256, 40, 8, 0.5), (64, 2880, 32, 4, 0.0),
                                          (300, 96, 256, 8, 1.0), (8192, 2880, 32, 4, 0.5)])
def test_route_topk_parity(T, H, E, k, bias):
    x, wr, br, lg, idx, w = _route(T, H, E, k, seed=31 + T, bias_std=bias)
    ref = oracle.router_logits(x, wr, br)
    assert np.all(np.abs(lg - ref) <= 1e-5 * (np.abs(ref) + 1) + 2e-6 * np.abs(ref).max()), \
        float(np.abs(lg - ref).max())
    oidx, ow = oracle.topk_softmax(lg, k)  # top-k on identical (GPU) logits
    np.testing.assert_array_equal(idx, oidx)
    np.testing.assert_allclose(w, ow, rtol=2e-6, atol=1e-7)
    # the oracle's own end-to-end routing agrees except where two logits are within noise
    ridx, _ = oracle.topk_softmax(ref, k)
    diff = np.any(ridx != idx, axis=1)
    for t in np.nonzero(diff)[0]:
        s = np.sort(ref[t])[::-1]
        assert np.min(np.abs(np.diff(s[:k + 1]))) < 1e-4, "routing differs beyond a near-tie"


# Routing inside mxfp4_moe_mlp: small batches with more than one expert group split H over 2 or
# 4 workgroups per tile, whose partial sums the selection kernel adds up in split order (T=64/E=32,
# T=100/E=32 and T=17/E=20: four splits, the latter with a ragged token tile and expert group;
# T=256/E=128: two; E=40: a ragged expert group). T=9/E=4 is one expert group: the logits
# kernel selects itself, no split. Large batches take the 64-token tiles over all experts with H split over S
# workgroups: T=8192/E=32 (2 expert blocks, S = 2) and T=4096/E=128 (8 blocks, S = 4) are the
# 20B and 120B prefill routers; T=600/E=256 (16 blocks, S = 8, ragged token tile), T=3000/E=40
# (4 blocks for 3 groups: a ragged block, S = 4 over 10 chunks: uneven splits) and
# T=9000/E=16 (1 block, H = 128: S = 1, logits and bias written by the tile kernel itself).
# Same bar as the router alone.
@pytest.mark.parametrize("T,H,E,k,bias", [(64, 2880, 32, 4, 0.0), (64, 2880, 40, 8, 0.5),
                                          (9, 3072, 4, 2, 0.5), (256, 2880, 128, 4, 1.0),
                                          (17, 2880, 20, 4, 0.5), (8192, 2880, 32, 4, 0.5),
                                          (4096, 2880, 128, 4, 1.0), (600, 1024, 256, 8, 1.0),
                                          (3000, 640, 40, 4, 0.5), (9000, 128, 16, 2, 0.5),
                                          (100, 2880, 32, 4, 0.5)])
def test_route_inside_moe_call(T, H, E, k, bias):
    seed, F = 35 + T, 64
    x = inputs.activations(seed, T, H)
    wr, br = inputs.router(seed, E, H, bias)
    note("route in moe call T=%d H=%d E=%d k=%d" % (T, H, E, k))
    _, (lg, idx, w) = mx.mxfp4_moe_mlp(to_dev(x), *moe_weights_dev(seed, E, H, F), k,
                                       wr=to_dev(wr), br=to_dev(br) if bias else None,
                                       out_dtype=torch.float32, return_routing=True)
    torch.cuda.synchronize()
    lg, idx, w = lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    ref = oracle.router_logits(x, wr, br if bias else None)
    assert np.all(np.abs(lg - ref) <= 1e-5 * (np.abs(ref) + 1) + 2e-6 * np.abs(ref).max()), \
        float(np.abs(lg - ref).max())
    oidx, ow = oracle.topk_softmax(lg, k)
    np.testing.assert_array_equal(idx, oidx)
    np.testing.assert_allclose(w, ow, rtol=2e-6, atol=1e-7)


def test_route_ties_go_to_lower_index():
    T, H, E, k = 20, 64, 16, 4
    wr = inputs.router(40, E, H)[0].copy()
    wr[5] = wr[2]       # experts 2 and 5 always tie
    wr[9] = wr[2]
    wr[11] = wr[7]
    x, wr, br, lg, idx, w = _route(T, H, E, k, seed=40, wr=wr)
    assert np.all(lg[:, 5] == lg[:, 2]) and np.all(lg[:, 9] == lg[:, 2])
    oidx, ow = oracle.topk_softmax(lg, k)
    np.testing.assert_array_equal(idx, oidx)
    x0 = np.zeros((3, H), np.uint16)   # zero tokens: all logits 0 -> experts 0..k-1, weights 1/k
    lg0, idx0, w0 = mx.moe_route_topk(to_dev(x0), to_dev(wr), None, k)
    torch.cuda.synchronize()
    assert np.all(idx0.cpu().numpy() == np.arange(k)) and np.all(w0.cpu().numpy() == 0.25)


def _permute(idx, E, use_workspace=False):
    """moe_permute (ws = NULL: one workgroup; else the sliced form for large batches); the
    fourth value is the device error word after the call (cleared before it)."""
    note("permute P=%d E=%d ws=%d" % (idx.size, E, use_workspace))
    assert mx.get_device_error() == 0
    offs, perm, inv = mx.moe_permute(to_dev(idx), E, use_workspace=use_workspace)
    st = mx.get_device_error()
    return offs.cpu().numpy(), perm.cpu().numpy(), inv.cpu().numpy(), st


@pytest.mark.parametrize("T,k,E,skew", [(1, 1, 1, 0), (1, 4, 128, 0), (3, 2, 8, 0),
                                        (64, 4, 32, 0), (1000, 3, 7, 1), (8192, 4, 32, 1),
                                        (4096, 4, 128, 0), (257, 8, 256, 0)])
def test_permute_bit_exact(T, k, E, skew):
    r = np.random.default_rng(50 + T)
    if skew:
        p = np.exp(r.normal(0, 1.5, E)); p /= p.sum()
        idx = np.stack([r.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    else:
        idx = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    offs, perm, inv, st = _permute(idx, E)
    o_offs, o_perm, o_inv = oracle.permute(idx, E)
    assert st == 0
    np.testing.assert_array_equal(offs, o_offs)
    np.testing.assert_array_equal(perm, o_perm)
    np.testing.assert_array_equal(inv, o_inv)


@pytest.mark.parametrize("T,k,E,skew,bad", [(2048, 4, 32, 0, 0), (8192, 4, 32, 1, 0),
                                            (4096, 4, 128, 0, 0), (10001, 3, 7, 1, 0),
                                            (3000, 8, 256, 1, 0), (5000, 4, 16, 0, 1),
                                            (5000, 8, 256, 1, 1)])
def test_permute_sliced_bit_exact(T, k, E, skew, bad):
    """moe_permute with its workspace: large batches go through the per-slice histogram and
    scatter (two launches, many workgroups); the result must be the oracle's counting sort
    element for element, and equal the one-workgroup form (ws = NULL). T=5000/k=8/E=256 has
    more slices (40) than one LDS chunk of slice histograms holds (31), with skipped indices in
    both chunks."""
    r = np.random.default_rng(70 + T)
    if skew:
        p = np.exp(r.normal(0, 1.5, E)); p /= p.sum()
        idx = np.stack([r.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    else:
        idx = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    if bad:  # a few indices outside [0, E), in different slices
        for pos in (5, 4100, 9000, T * k - 1):
            idx.reshape(-1)[pos] = E + 3 if pos % 2 else -2
    offs, perm, inv, st = _permute(idx, E, use_workspace=True)
    assert st == (mx.MX_DEVERR_ROUTING if bad else 0)
    if not bad:
        o_offs, o_perm, o_inv = oracle.permute(idx, E)
        np.testing.assert_array_equal(offs, o_offs)
        np.testing.assert_array_equal(perm, o_perm)
        np.testing.assert_array_equal(inv, o_inv)
    # the one-workgroup path gives the same arrays (including skipped pairs)
    o1, p1, i1, s1 = _permute(idx, E)
    assert s1 == st
    n = int(offs[-1])
    np.testing.assert_array_equal(offs, o1)
    np.testing.assert_array_equal(perm[:n], p1[:n])
    np.testing.assert_array_equal(inv, i1)


def test_permute_all_to_one_expert_and_empty_experts():
    idx = np.full((500, 1), 3, np.int32)
    offs, perm, inv, st = _permute(idx, 9)
    o = oracle.permute(idx, 9)
    np.testing.assert_array_equal(offs, o[0])
    np.testing.assert_array_equal(perm, o[1])
    np.testing.assert_array_equal(inv, o[2])


def test_permute_flags_out_of_range_indices():
    idx = np.array([[0, 1], [5, 2], [-1, 0]], np.int32)
    offs, perm, inv, st = _permute(idx, 4)
    assert st == mx.MX_DEVERR_ROUTING
    assert mx.get_device_error() == 0  # reading clears the word
    assert inv[2] == -1 and inv[4] == -1
    valid = np.array([0, 1, 3, 5])  # pairs with an index inside [0, 4)
    assert offs[-1] == 4 and sorted(perm[:4].tolist()) == valid.tolist()
    np.testing.assert_array_equal(perm[:4], [0, 5, 1, 3])  # experts 0,0,1,2 in pair order


@pytest.mark.parametrize("T,H,E,k,bias", [(1, 2880, 128, 4, 0.0), (64, 2880, 32, 4, 0.5),
                                          (37, 256, 40, 8, 0.5), (300, 96, 256, 8, 1.0)])
def test_route_topk_without_logits(T, H, E, k, bias):
    """logits = NULL: the workgroups cover all experts of their tokens and select from on-chip
    memory (another split of H than with a logits buffer, so the fp32 sums may differ in the
    last bits): indices equal the oracle's top-k except where two oracle logits are within fp32
    noise, and the weights match the oracle's softmax."""
    seed = 90 + T
    x = inputs.activations(seed, T, H)
    wr, br = inputs.router(seed, E, H, bias)
    br = br if bias else None
    note("route without logits T=%d H=%d E=%d k=%d" % (T, H, E, k))
    lg, idx, w = mx.moe_route_topk(to_dev(x), to_dev(wr), None if br is None else to_dev(br), k,
                                   want_logits=False)
    torch.cuda.synchronize()
    assert lg is None
    idx, w = idx.cpu().numpy(), w.cpu().numpy()
    ref = oracle.router_logits(x, wr, br)
    oidx, ow = oracle.topk_softmax(ref, k)
    same = np.all(idx == oidx, axis=1)
    for t in np.nonzero(~same)[0]:
        s = np.sort(ref[t])[::-1]
        assert np.min(np.abs(np.diff(s[:k + 1]))) < 1e-4, "routing differs beyond a near-tie"
    np.testing.assert_allclose(w[same], ow[same], rtol=2e-5, atol=1e-6)
