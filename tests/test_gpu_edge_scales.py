"""GPU: extreme E8M0 scale bytes (0, 1, 2, 253, 254, 255) with all 16 codes through the matrix
products of mxfp4_linear and mxfp4_moe_mlp, bf16 path and activation variant, against the
oracle.

Reading checked here (the weight operand): with bf16 activations a weight enters the product as
the bf16 value of code * 2^(b-127) -- exact, subnormals included, except past bf16's largest
finite number, where it is +-Inf; byte 255 is NaN; products and sums follow IEEE arithmetic, so
Inf and NaN propagate and subnormal results are kept. The activation variant multiplies the MXFP4
values exactly (a weight of 6 * 2^127 stays finite there). Accumulation is fp32 on both paths, so
the inputs keep every running sum inside fp32's range (no case where an fp32 partial sum would
overflow and the exact total would not).

Weights are built by hand as packed bytes; activations are drawn at magnitudes that put the
products in range: N(0,1) times 2^100 against the tiny scales, times 2^-120 (or 2^-100) against
the huge ones."""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_weight_quantized_amd import inputs
import mxfp4_weight_quantized_amd as mx
from parity_util import (FRAGILE_C, check_tolerance_nonfinite, note, tiled_dev, to_dev, to_f64)

pytestmark = pytest.mark.gpu

MX = mx.MX_ACT_MXFP4
TINY = (0, 1, 2)
HUGE = (253, 254)
# codes whose value times 2^(b-127) bf16 holds: |v| <= 3 at byte 253, |v| <= 1.5 at byte 254
FINITE = {253: [c for c in range(16) if (c & 7) <= 5], 254: [c for c in range(16) if (c & 7) <= 3]}


def _pack(codes):
    codes = np.asarray(codes, np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _block_codes(r, byte):
    """32 codes of one block: every allowed code at least once, the rest drawn from them."""
    allowed = np.array(FINITE.get(byte, list(range(16))))
    c = np.concatenate([allowed, r.choice(allowed, size=32 - len(allowed))])
    return r.permutation(c)


def _rows(r, n, K, kind):
    """n weight rows [n][K] of one kind as (codes, scale bytes)."""
    nb = K // 32
    codes = np.zeros((n, K), np.uint8)
    sb = np.zeros((n, nb), np.uint8)
    for i in range(n):
        for b in range(nb):
            if kind == "tiny":
                byte = int(r.choice(TINY))
            elif kind == "huge":
                byte = int(r.choice(HUGE))
            elif kind == "mixed":
                byte = int(r.choice(TINY + (127,) + HUGE))
            else:  # "normal" surroundings of the Inf / NaN rows
                byte = int(r.integers(118, 123))
            sb[i, b] = byte
            codes[i, 32 * b:32 * b + 32] = _block_codes(r, byte)
        if kind == "inf_one":    # one element 6 * 2^127 (+-), the rest of its block zero
            b = int(r.integers(nb))
            codes[i, 32 * b:32 * b + 32] = 0
            codes[i, 32 * b + int(r.integers(32))] = 7 if i % 2 == 0 else 15
            sb[i, b] = 254
        elif kind == "inf_block":  # a byte-254 block with all 16 codes: +Inf and -Inf weights
            b = int(r.integers(nb))
            codes[i, 32 * b:32 * b + 32] = r.permutation(np.tile(np.arange(16), 2))
            sb[i, b] = 254
        elif kind == "nan":
            sb[i, int(r.integers(nb))] = 255
    return codes, sb


def _weight(r, K, kinds, n_per=24):
    parts = [_rows(r, n_per, K, k) for k in kinds]
    codes = np.concatenate([c for c, _ in parts])
    sb = np.concatenate([s for _, s in parts])
    return _pack(codes), sb


def _x(seed, M, K, log2_scale):
    """bf16 activations N(0, 1) * 2^log2_scale."""
    a = inputs.normal_f32(seed, inputs.TAG_MISC, (M, K), 1.0, sub=1000 + log2_scale)
    return inputs.bf16_bits(np.ldexp(a, log2_scale).astype(np.float32))


# (x magnitude 2^e, weight row kinds, paths) -- each call keeps every fp32 partial sum in range
LINEAR_CASES = [
    (100, ("tiny",), (0, MX)),                      # products ~2^-27
    (0, ("tiny",), (0, MX)),                        # products ~2^-127: subnormal fp32 results
    (-120, ("huge",), (0, MX)),                     # products ~2^7
    (-120, ("mixed",), (0, MX)),                    # tiny terms vanish next to the huge ones
    (-120, ("inf_one", "inf_block"), (0, MX)),      # bf16: +-Inf / NaN; activation variant: finite
    (0, ("inf_one", "inf_block", "nan"), (0,)),     # bf16 path: Inf and NaN patterns
    (0, ("nan",), (MX,)),                           # NaN scale: NaN on both paths
]


@pytest.mark.parametrize("M,K", [(1, 1024), (5, 96), (80, 1024)])
@pytest.mark.parametrize("case", range(len(LINEAR_CASES)))
def test_linear_extreme_scale_bytes(case, M, K):
    e, kinds, paths = LINEAR_CASES[case]
    r = np.random.default_rng(1000 + 10 * case + M)
    p, s = _weight(r, K, kinds)
    x = _x(40 + case, M, K, e)
    for flags in paths:
        note("linear extreme scales case %d (x 2^%d, %s) M=%d K=%d flags=%d" % (
            case, e, "+".join(kinds), M, K, flags))
        y = mx.mxfp4_linear(to_dev(x), to_dev(p), to_dev(s), out_dtype=torch.float32, flags=flags)
        torch.cuda.synchronize()
        ref = oracle.linear(x, p, s, mx_act=bool(flags))
        check_tolerance_nonfinite(to_f64(y), ref, "linear case %d flags=%d" % (case, flags))


# ------------------------------------------------------------------------------------ MoE MLP
H = F = 64
# expert e: (gate_up row kind, down row kind, log2 of its tokens' activation scale)
EXPERTS = [
    ("tiny", "normal", 100),      # e0: g, u ~ 2^-23
    ("normal", "tiny", 0),        # e1: outputs ~2^-130 (subnormal fp32)
    ("huge", "normal", -100),     # e2
    ("normal", "huge", -40),      # e3: h ~ 2^-87, outputs ~2^43
    ("inf_one", "normal", -100),  # e4: one +-6 * 2^127 weight in every gate row
    ("normal", "inf_one", -40),   # e5: one +-6 * 2^127 weight in every down row
    ("normal", "nan", 0),         # e6: a NaN-scale block in every down row
    ("normal", "normal", 0),      # e7
]
E = len(EXPERTS)


def _normal_rows(seed, n, K):
    return oracle.quantize(inputs.normal_f32(seed, inputs.TAG_MISC, (n, K), 0.02, sub=n * K))


def _moe_weights(seed):
    r = np.random.default_rng(seed)
    gp = np.zeros((E, 2 * F, H // 2), np.uint8)
    gs = np.zeros((E, 2 * F, H // 32), np.uint8)
    dp = np.zeros((E, H, F // 2), np.uint8)
    ds = np.zeros((E, H, F // 32), np.uint8)
    for e, (gk, dk, _) in enumerate(EXPERTS):
        if gk == "normal":
            gp[e], gs[e] = _normal_rows(seed + e, 2 * F, H)
        elif gk == "inf_one":  # the special element in gate rows only; up rows normal
            gp[e], gs[e] = _normal_rows(seed + e, 2 * F, H)
            c, sb = _rows(r, F, H, "inf_one")
            for i in range(F):
                blk = int(np.nonzero(sb[i] == 254)[0][0])
                row = np.zeros(H, np.uint8)
                row[0::2], row[1::2] = gp[e, i] & 15, gp[e, i] >> 4
                row[32 * blk:32 * blk + 32] = c[i, 32 * blk:32 * blk + 32]
                gp[e, i] = _pack(row)
                gs[e, i, blk] = 254
        else:
            c, sb = _rows(r, 2 * F, H, gk)
            gp[e], gs[e] = _pack(c), sb
        if dk == "normal":
            dp[e], ds[e] = _normal_rows(seed + 50 + e, H, F)
        elif dk == "nan":
            dp[e], ds[e] = _normal_rows(seed + 50 + e, H, F)
            ds[e, :, int(r.integers(F // 32))] = 255
        else:
            c, sb = _rows(r, H, F, dk)
            dp[e], ds[e] = _pack(c), sb
    return gp, gs, dp, ds


def _moe_tokens(seed, per_expert, k):
    """Tokens grouped by activation scale; k = 1: one expert each; k = 2: pairs of experts that
    take the same scale."""
    if k == 1:
        groups = [([e], EXPERTS[e][2]) for e in range(E)]
    else:
        groups = [([1, 7], 0), ([6, 7], 0), ([1, 6], 0), ([2, 4], -100), ([3, 5], -40)]
    xs, idx, w = [], [], []
    r = np.random.default_rng(seed)
    for gi, (experts, e2) in enumerate(groups):
        xs.append(_x(seed + gi, per_expert, H, e2))
        for _ in range(per_expert):
            idx.append(r.permutation(experts)[:k])
    x = np.concatenate(xs)
    idx = np.array(idx, np.int32)
    w = r.uniform(0.1, 1.0, size=idx.shape).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    return x, idx, w


# per_expert 3 / 5: decode-shaped tiles; 70 (k = 1: 560 pairs >= 64 E) and 130 (k = 2: 1300
# pairs): prefill-shaped tiles
@pytest.mark.parametrize("per_expert,k", [(3, 1), (70, 1), (5, 2), (130, 2)])
@pytest.mark.parametrize("flags", [0, MX])
def test_moe_extreme_scale_bytes(per_expert, k, flags):
    seed = 2000 + per_expert + 10 * k
    wts = _moe_weights(seed)
    x, idx, w = _moe_tokens(seed, per_expert, k)
    note("moe extreme scales T=%d k=%d flags=%d" % (x.shape[0], k, flags))
    wd = tuple(to_dev(a) for a in wts)
    xd, idxd, wdv = to_dev(x), to_dev(idx), to_dev(w)
    out = mx.mxfp4_moe_mlp(xd, *wd, k, topk_idx=idxd, topk_w=wdv, out_dtype=torch.float32,
                           flags=flags)
    out_t = mx.mxfp4_moe_mlp(xd, *tiled_dev(wd), k, topk_idx=idxd, topk_w=wdv,
                             out_dtype=torch.float32, flags=flags | mx.MX_WEIGHTS_TILED)
    torch.cuda.synchronize()
    a, b = to_f64(out), to_f64(out_t)
    np.testing.assert_array_equal(np.isnan(a), np.isnan(b))
    np.testing.assert_array_equal(np.where(np.isnan(a), 0, a), np.where(np.isnan(b), 0, b))
    if flags & MX:
        ref, _, slack = oracle.moe_mlp(x, idx, w, *wts, E=E, mx_act=True, fragile_c=FRAGILE_C)
    else:
        ref, slack = oracle.moe_mlp(x, idx, w, *wts, E=E), None
    check_tolerance_nonfinite(a, ref, "moe extreme scales flags=%d" % flags, slack=slack)
    # the cases do reach the regimes they are meant to: NaN (NaN scales), +-Inf (bf16 path:
    # overflowing weights), and with one expert per token subnormal and very large outputs
    assert np.isnan(ref).any()
    assert np.isinf(ref).any() == (not flags)
    if k == 1:
        fin = np.abs(ref[np.isfinite(ref)])
        assert (fin[fin > 0] < 2.0 ** -126).any() and (fin > 2.0 ** 40).any()
