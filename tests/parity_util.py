"""Helpers shared by the GPU parity tests: tolerance checks, tensor moves, cached weights.

Inputs come from the seeded generators in mxfp4_weight_quantized_amd.inputs; packed weights
used as inputs of the GPU path are produced by the oracle's quantizer (never by the GPU).
"""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
from mxfp4_weight_quantized_amd import inputs

DEV = "cuda:0"

# MoE-MLP / linear output tolerance: relative Frobenius error and a per-element bound scaled by
# the root-mean-square of the oracle's output row.
REL_FROB = 5e-3
PER_ELEM = 1e-2
PER_ELEM_FLOOR = 1e-3


def note(msg: str):
    """Progress line that bypasses pytest's capture (names the case before a GPU step)."""
    sys.__stdout__.write("[gpu] %s\n" % msg)
    sys.__stdout__.flush()


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    """numpy -> device tensor. uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    t = t.to(DEV)
    return t if dtype is None else t.to(dtype)


def bf16_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").view(torch.int16).numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_tolerance(got: np.ndarray, ref: np.ndarray, what: str = "", slack=None):
    """Output bound: ||got-ref||_F <= 5e-3 ||ref||_F and, per element,
    |got-ref| <= 1e-2 * (||ref row||_2 / sqrt(N) + 1e-3).
    slack (activation variant): per-element allowance for the h quantization decisions the oracle
    flagged as fragile; the error is reduced by it (not below 0) before both checks."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    err = got - ref
    if slack is not None:
        err = np.sign(err) * np.maximum(np.abs(err) - np.asarray(slack, np.float64), 0.0)
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= REL_FROB, "%s: relative Frobenius error %.3e" % (what, rel)
    rms = np.linalg.norm(ref, axis=-1, keepdims=True) / np.sqrt(ref.shape[-1])
    bound = PER_ELEM * (rms + PER_ELEM_FLOOR)
    bad = np.abs(err) > bound
    assert not bad.any(), "%s: %d elements over the per-element bound (max ratio %.3f)" % (
        what, int(bad.sum()), float((np.abs(err) / bound).max()))
    return rel


def _bf16_rne(a: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 value (ties to even) through torch's cast, as fp64."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float64)).to(torch.bfloat16).double().numpy()


def check_bf16_output(got_bits: np.ndarray, ref: np.ndarray, what: str = "", slack=None,
                      got_f32=None):
    """bf16 output. The output is the bf16 rounding of the path's fp32 result, so it passes when
    it is the bf16 rounding of some value within the output bound of the oracle's value:
    rounding is monotone, so per element RNE(ref - b) <= got <= RNE(ref + b) with
    b = 1e-2 (||ref row|| / sqrt(N) + 1e-3) (+ the fragile-decision slack, if given). The
    relative Frobenius error must stay within 5e-3. With got_f32 (the same call's fp32 output)
    the bf16 output must also be exactly its round-to-nearest-even bf16."""
    got = inputs.bf16_to_f32(got_bits).astype(np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    if got_f32 is not None:
        np.testing.assert_array_equal(got, _bf16_rne(np.asarray(got_f32, np.float64)),
                                      err_msg="%s: bf16 output is not RNE of the fp32 output" % what)
    rms = np.linalg.norm(ref, axis=-1, keepdims=True) / np.sqrt(ref.shape[-1])
    b = PER_ELEM * (rms + PER_ELEM_FLOOR) + (0.0 if slack is None else np.asarray(slack, np.float64))
    lo, hi = _bf16_rne(ref - b), _bf16_rne(ref + b)
    bad = (got < lo) | (got > hi)
    assert not bad.any(), "%s: %d bf16 elements outside the rounded output bound" % (
        what, int(bad.sum()))
    err = got - ref
    if slack is not None:
        err = np.sign(err) * np.maximum(np.abs(err) - np.asarray(slack, np.float64), 0.0)
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= REL_FROB, "%s: relative Frobenius error %.3e" % (what, rel)


@functools.lru_cache(maxsize=4)
def moe_weights(seed: int, E: int, H: int, F: int):
    """Oracle-packed expert weights for a (seed, E, H, F) layer, on the host (random draws on
    worker threads, the oracle's quantizer on this thread)."""
    return inputs.expert_weights(seed, E, H, F, oracle.quantize, threads=8)


@functools.lru_cache(maxsize=4)
def moe_weights_dev(seed: int, E: int, H: int, F: int):
    return tuple(to_dev(a) for a in moe_weights(seed, E, H, F))


# ----------------------------------------------------------------------------------------------
# Full-size layers: one oracle run per layer, routed by the oracle's own router
# ----------------------------------------------------------------------------------------------
ROUTE_TOL = 1e-5   # GPU logits vs the oracle's: |d| <= 1e-5 (|l| + 1) (fp32 vs fp64 sums)
FRAGILE_C = 4.0    # activation variant: assumed fp32 error of g and u, 4 * 2^-24 * sqrt(H sum t^2)


@functools.lru_cache(maxsize=8)
def oracle_layer(shape):
    """(x, wr, br, logits, idx, w) of a MoE layer shape, routed by the oracle (fp64 logit sums,
    rounded to fp32; top-k and softmax on those)."""
    s = shape
    x = inputs.activations(s.seed, s.T, s.H)
    wr, br = inputs.router(s.seed, s.E, s.H, s.bias_std)
    br = br if s.bias_std else None
    lg = oracle.router_logits(x, wr, br)
    idx, w = oracle.topk_softmax(lg, s.k)
    return x, wr, br, lg, idx, w


@functools.lru_cache(maxsize=3)
def layer_weights(seed: int, E: int, H: int, F: int):
    """Oracle-packed weights of a full-size layer (cached apart from the small test layers)."""
    return inputs.expert_weights(seed, E, H, F, oracle.quantize, threads=8)


@functools.lru_cache(maxsize=3)
def layer_weights_dev(seed: int, E: int, H: int, F: int):
    return tuple(to_dev(a) for a in layer_weights(seed, E, H, F))


@functools.lru_cache(maxsize=16)
def oracle_output(shape, mx_act: bool):
    """The oracle's MoE output for every token of the layer under its own routing (fp64 rows),
    and for the activation variant the fragile-decision slack (else None)."""
    x, _, _, _, idx, w = oracle_layer(shape)
    wts = layer_weights(shape.seed, shape.E, shape.H, shape.F)
    note("oracle: %s%s, %d tokens" % (shape.name, " (activation variant)" if mx_act else "",
                                       shape.T))
    if mx_act:
        out, _, slack = oracle.moe_mlp(x, idx, w, *wts, E=shape.E, mx_act=True,
                                       fragile_c=FRAGILE_C)
        return out, slack
    return oracle.moe_mlp(x, idx, w, *wts, E=shape.E), None


def routing_parity(shape, g_lg, g_idx, g_w):
    """Checks the GPU router's outputs for a layer and returns the tokens whose GPU routing
    differs from the oracle's own (each shown to be a near-tie the fp32 logits may order either
    way), with the oracle's routing for them (idx, w) over the experts the GPU chose.
      - logits within ROUTE_TOL (|l| + 1) of the oracle's, plus 2e-6 of the largest |logit|
        (fp32 sums of H = 2880 products);
      - indices bit-exact, and weights to 2e-6, against the oracle's top-k and softmax over the
        GPU's own logits (the selection is exact given the logits);
      - where the GPU's expert set or order differs from the oracle's, every expert involved has
        an oracle logit within the sum of the two logits' tolerances of the one it displaced."""
    _, _, _, o_lg, o_idx, _ = oracle_layer(shape)
    k = shape.k
    g_lg, g_idx, g_w = (np.asarray(a) for a in (g_lg, g_idx, g_w))
    ref = o_lg.astype(np.float64)
    d = np.abs(g_lg.astype(np.float64) - ref)
    assert np.all(d <= ROUTE_TOL * (np.abs(ref) + 1) + 2e-6 * np.abs(ref).max()), \
        "router logits off by up to %.3e" % d.max()
    sel_idx, sel_w = oracle.topk_softmax(g_lg, k)
    np.testing.assert_array_equal(g_idx, sel_idx)
    np.testing.assert_allclose(g_w, sel_w, rtol=2e-6, atol=1e-7)
    ties = np.nonzero((g_idx != o_idx).any(axis=1))[0].astype(np.int32)
    t_idx = np.zeros((len(ties), k), np.int32)
    t_w = np.zeros((len(ties), k), np.float32)
    for n, t in enumerate(ties):
        row = o_lg[t].astype(np.float64)
        for j in range(k):
            a, b = row[g_idx[t, j]], row[o_idx[t, j]]
            if g_idx[t, j] != o_idx[t, j]:
                assert abs(a - b) <= ROUTE_TOL * (abs(a) + abs(b) + 2), \
                    "token %d: routing differs beyond a near-tie" % t
        masked = np.full((1, shape.E), -np.inf, np.float32)
        masked[0, g_idx[t]] = o_lg[t, g_idx[t]]
        ti, tw = oracle.topk_softmax(masked, k)
        t_idx[n], t_w[n] = ti[0], tw[0]
    if len(ties):
        note("%s: %d near-tie tokens routed differently" % (shape.name, len(ties)))
    return ties, t_idx, t_w


def full_reference(shape, mx_act: bool, ties, t_idx, t_w):
    """Oracle output (and slack) for every token; near-tie tokens recomputed under the GPU's
    (validated) expert choice."""
    out, slack = oracle_output(shape, mx_act)
    if len(ties) == 0:
        return out, slack
    out, slack = out.copy(), None if slack is None else slack.copy()
    x = oracle_layer(shape)[0]
    wts = layer_weights(shape.seed, shape.E, shape.H, shape.F)
    idx = np.zeros((shape.T, shape.k), np.int32)
    w = np.zeros((shape.T, shape.k), np.float32)
    idx[ties], w[ties] = t_idx, t_w
    if mx_act:
        o, _, sl = oracle.moe_mlp(x, idx, w, *wts, E=shape.E, tokens=ties, mx_act=True,
                                  fragile_c=FRAGILE_C)
        slack[ties] = sl
    else:
        o = oracle.moe_mlp(x, idx, w, *wts, E=shape.E, tokens=ties)
    out[ties] = o
    return out, slack


def tiled_dev(wdev):
    """The grouped GEMMs' tiled layout of device weights (mxfp4_tile_weights)."""
    import mxfp4_weight_quantized_amd as mx
    gp, gs, dp, ds = wdev
    return (*mx.mxfp4_tile_weights(gp, gs), *mx.mxfp4_tile_weights(dp, ds))


def run_full_layer(shape, flags: int, out_dtype, tiled: bool):
    """The whole MoE MLP on the GPU with internal routing; returns (out, logits, idx, w) on the
    host (out: fp64 for fp32 outputs, bf16 bits for bf16 outputs)."""
    import mxfp4_weight_quantized_amd as mx
    s = shape
    x, wr, br, _, _, _ = oracle_layer(s)
    wd = layer_weights_dev(s.seed, s.E, s.H, s.F)
    if tiled:
        wd = tiled_dev(wd)
        flags |= mx.MX_WEIGHTS_TILED
    note("moe full %s flags=%d %s" % (s.name, flags, out_dtype))
    out, (lg, idx, w) = mx.mxfp4_moe_mlp(
        to_dev(x), *wd, s.k, wr=to_dev(wr), br=None if br is None else to_dev(br),
        out_dtype=out_dtype, flags=flags, return_routing=True)
    torch.cuda.synchronize()
    got = to_f64(out) if out_dtype == torch.float32 else bf16_host_bits(out)
    return got, lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def check_full_layer(shape, flags: int = 0, tiled: bool = False, out_dtypes=None):
    """Every token of a full-size layer against one oracle run, for each output dtype."""
    import mxfp4_weight_quantized_amd as mx
    mx_act = bool(flags & mx.MX_ACT_MXFP4)
    got32 = None
    for out_dtype in (out_dtypes or (torch.float32, torch.bfloat16)):
        got, lg, idx, w = run_full_layer(shape, flags, out_dtype, tiled)
        ties, t_idx, t_w = routing_parity(shape, lg, idx, w)
        ref, slack = full_reference(shape, mx_act, ties, t_idx, t_w)
        what = "%s flags=%d tiled=%d %s" % (shape.name, flags, tiled, out_dtype)
        if out_dtype == torch.float32:
            check_tolerance(got, ref, what, slack=slack)
            got32 = got
        else:
            check_bf16_output(got, ref, what, slack=slack, got_f32=got32)


def check_tolerance_nonfinite(got, ref, what="", slack=None, scale_free=True):
    """Outputs where the weights reach past fp32/bf16's range or hold NaN scales. The fp64
    reference is first rounded to the fp32 output (its precision point: values past fp32's range
    are +-Inf there, values below it 0 or subnormal). Then: NaN exactly where the reference is
    NaN, +-Inf exactly where it is +-Inf (same sign); the finite elements meet the output bound
    with row norms over each row's finite elements, and (scale_free) also |err| <= 1e-2 * row rms
    without the absolute floor, so rows of tiny values are held to the same relative bound as
    the others."""
    got = np.asarray(got, np.float64)
    with np.errstate(over="ignore"):
        ref = np.asarray(ref, np.float64).astype(np.float32).astype(np.float64)
    assert got.shape == ref.shape
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref), err_msg="%s: NaN positions" % what)
    inf = np.isinf(ref)
    np.testing.assert_array_equal(np.isinf(got), inf, err_msg="%s: Inf positions" % what)
    assert np.all(np.sign(got[inf]) == np.sign(ref[inf])), "%s: Inf signs" % what
    fin = np.isfinite(ref)
    err = np.where(fin, got - ref, 0.0)
    if slack is not None:
        sl = np.where(fin, np.asarray(slack, np.float64), 0.0)
        err = np.sign(err) * np.maximum(np.abs(err) - sl, 0.0)
    r0 = np.where(fin, ref, 0.0)
    nfin = np.maximum(fin.sum(axis=-1, keepdims=True), 1)
    rms = np.linalg.norm(r0, axis=-1, keepdims=True) / np.sqrt(nfin)
    bound = PER_ELEM * (rms + PER_ELEM_FLOOR)
    bad = (np.abs(err) > bound) & fin
    assert not bad.any(), "%s: %d finite elements over the per-element bound" % (what, int(bad.sum()))
    if scale_free:
        bad = (np.abs(err) > PER_ELEM * rms) & fin
        assert not bad.any(), "%s: %d finite elements over 1e-2 x row rms (max ratio %.3g)" % (
            what, int(bad.sum()), float((np.abs(err) / np.maximum(PER_ELEM * rms, 1e-300))[fin].max()))
    for i in range(ref.shape[0]):  # relative Frobenius error per row of finite values
        f = fin[i]
        nr = np.linalg.norm(ref[i][f])
        if nr > 0:
            rel = np.linalg.norm(err[i][f]) / nr
            assert rel <= REL_FROB, "%s: row %d relative Frobenius error %.3e" % (what, i, rel)
