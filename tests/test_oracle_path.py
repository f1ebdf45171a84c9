"""Pins for the oracle's router, permutation, dense linear and MoE MLP (CPU only).

References used here are independent of the oracle's C code: numpy fp64 matrix products on
weights decoded with the golden value table, Python's stable ``sorted``, torch's bf16 cast, and
special cases that reduce the MoE MLP to a dense SwiGLU MLP.
"""
import os

import numpy as np
import pytest

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


def _decode_np(packed, scales, tab):
    """Independent numpy decode: nibbles (low first) -> table -> times 2^(byte-127)."""
    packed = np.asarray(packed)
    codes = np.stack([packed & 15, packed >> 4], axis=-1).reshape(*packed.shape[:-1], -1)
    sc = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)
    return tab[codes] * sc


def _bf16_f64(bits):
    return inputs.bf16_to_f32(bits).astype(np.float64)


def _bf16_round(a64):
    torch = pytest.importorskip("torch")
    # values here are exactly representable in fp32 up to the last fp64 bits; route via fp32 is
    # the library's own single cast on fp32-exact inputs, so compare with tolerance of 1 bf16 ulp
    return torch.from_numpy(a64.astype(np.float32)).to(torch.bfloat16).float().double().numpy()


# ---------------------------------------------------------------------------------------------
def test_linear_matches_numpy_bruteforce(golden_dir):
    tab = _table(golden_dir)
    M, K, N = 3, 96, 5
    x = inputs.activations(11, M, K)
    w = inputs.normal_f32(11, inputs.TAG_MISC, (N, K), 0.02)
    p, s = oracle.quantize(w)
    y = oracle.linear(x, p, s)
    ref = _bf16_f64(x) @ _decode_np(p, s, tab).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-15)
    # a transposed operand or swapped roles would not match at these non-square shapes
    assert y.shape == (M, N)


def test_linear_mx_act_k32_is_exact_and_uses_quantized_x(golden_dir):
    """Activation variant: x is quantized like the weights; with K = 32 every product is a power of
    two times a multiple of 1/4, so the fp64 sum is exact."""
    tab = _table(golden_dir)
    M, K, N = 4, 32, 7
    x = inputs.activations(12, M, K)
    w = inputs.normal_f32(12, inputs.TAG_MISC, (N, K), 0.02)
    p, s = oracle.quantize(w)
    xp, xs = oracle.quantize(x)
    y = oracle.linear(x, p, s, mx_act=True)
    ref = _decode_np(xp, xs, tab) @ _decode_np(p, s, tab).T
    np.testing.assert_array_equal(y, ref)
    y_plain = oracle.linear(x, p, s, mx_act=False)
    assert not np.array_equal(y_plain, y)


# ---------------------------------------------------------------------------------------------
def test_router_logits_match_numpy():
    T, H, E = 9, 64, 6
    x = inputs.activations(13, T, H)
    wr, br = inputs.router(13, E, H, bias_std=0.5)
    lg = oracle.router_logits(x, wr, br)
    ref = (_bf16_f64(x) @ _bf16_f64(wr).T + br.astype(np.float64)).astype(np.float32)
    np.testing.assert_allclose(lg, ref, rtol=2 ** -23, atol=0)
    lg0 = oracle.router_logits(x, wr, None)
    ref0 = (_bf16_f64(x) @ _bf16_f64(wr).T).astype(np.float32)
    np.testing.assert_allclose(lg0, ref0, rtol=2 ** -23, atol=0)


def test_topk_matches_sorted_and_softmax_properties():
    r = np.random.default_rng(14)
    T, E = 200, 32
    logits = r.standard_normal((T, E)).astype(np.float32)
    logits[:20] = np.round(logits[:20])  # many equal logits: the tie rule matters
    for k in (1, 2, 4, 8):
        idx, w = oracle.topk_softmax(logits, k)
        for t in range(T):
            want = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
            assert list(idx[t]) == want
            sel = logits[t, want].astype(np.float64)
            ref = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
            np.testing.assert_allclose(w[t], ref, rtol=1e-6)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
        if k == 1:
            assert np.all(w == 1.0)


def test_topk_all_equal_logits():
    idx, w = oracle.topk_softmax(np.zeros((3, 16), np.float32), 4)
    assert np.all(idx == np.arange(4)) and np.all(w == 0.25)


# ---------------------------------------------------------------------------------------------
def _check_perm(idx, E, offsets, perm, inv):
    T, k = idx.shape
    flat = idx.reshape(-1)
    want = sorted(range(T * k), key=lambda p: flat[p])  # Python's sort is stable
    assert list(perm) == want
    assert offsets[0] == 0 and offsets[E] == T * k
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
    assert np.array_equal(perm[inv], np.arange(T * k))
    assert np.array_equal(inv[perm], np.arange(T * k))


def test_permute_matches_stable_sort():
    r = np.random.default_rng(15)
    for T, k, E in [(1, 1, 1), (1, 4, 8), (37, 4, 32), (100, 2, 5), (64, 8, 256)]:
        idx = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        offsets, perm, inv = oracle.permute(idx, E)
        _check_perm(idx, E, offsets, perm, inv)


def test_permute_skewed_and_empty_experts():
    T, k, E = 50, 1, 10
    idx = np.full((T, k), 7, np.int32)  # every token to one expert; the others stay empty
    offsets, perm, inv = oracle.permute(idx, E)
    assert list(offsets) == [0] * 8 + [50] * 3
    _check_perm(idx, E, offsets, perm, inv)
    with pytest.raises(ValueError):
        oracle.permute(np.array([[E]], np.int32), E)


# ---------------------------------------------------------------------------------------------
def _small_moe(seed, T, H, F, E, k):
    x = inputs.activations(seed, T, H)
    gu_p, gu_s, dn_p, dn_s = inputs.expert_weights(seed, E, H, F, oracle.quantize, threads=2)
    return x, gu_p, gu_s, dn_p, dn_s


def _dense_swiglu(x64, wgu, wdn, F):
    a = x64 @ wgu.T
    g, u = a[:, :F], a[:, F:]
    h = _bf16_round(g / (1 + np.exp(-g)) * u)
    return h, h @ wdn.T


def test_moe_single_expert_is_dense_swiglu_mlp(golden_dir):
    """E = 1, k = 1: routing weight 1, so the MoE MLP is silu(x Wg^T) * (x Wu^T) -> bf16 -> Wd."""
    tab = _table(golden_dir)
    T, H, F = 6, 64, 96
    x, gu_p, gu_s, dn_p, dn_s = _small_moe(16, T, H, F, 1, 1)
    idx = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    out, h = oracle.moe_mlp(x, idx, w, gu_p, gu_s, dn_p, dn_s, E=1, want_h=True)
    href, ref = _dense_swiglu(_bf16_f64(x), _decode_np(gu_p[0], gu_s[0], tab),
                              _decode_np(dn_p[0], dn_s[0], tab), F)
    hgot = _bf16_f64(h[:, 0, :])
    # bf16 rounding from fp64 vs from fp32 may differ by one ulp on rare elements
    assert np.mean(hgot != href) < 0.01
    np.testing.assert_allclose(hgot, href, rtol=2 ** -7, atol=1e-30)
    ref_from_h = hgot @ _decode_np(dn_p[0], dn_s[0], tab).T
    np.testing.assert_allclose(out, ref_from_h, rtol=1e-11, atol=1e-14)
    # secondary, loose check of the whole chain against numpy (the exact pin is the line above):
    # numpy's h is rounded to bf16 through fp32, so a few h elements may sit one bf16 ulp
    # (2^-8 relative) away from the oracle's, and each such flip moves the outputs a little
    np.testing.assert_allclose(out, ref, rtol=2e-2, atol=1e-3)


def test_moe_all_experts_weighted_sum(golden_dir):
    """k = E: every expert contributes, weighted by the full softmax of the logits."""
    tab = _table(golden_dir)
    T, H, F, E = 5, 32, 64, 3
    x, gu_p, gu_s, dn_p, dn_s = _small_moe(17, T, H, F, E, E)
    wr, br = inputs.router(17, E, H, bias_std=1.0)
    idx, w = oracle.topk_softmax(oracle.router_logits(x, wr, br), E)
    out = oracle.moe_mlp(x, idx, w, gu_p, gu_s, dn_p, dn_s, E=E)
    ref = np.zeros((T, H))
    x64 = _bf16_f64(x)
    for t in range(T):
        for j in range(E):
            e = idx[t, j]
            _, y = _dense_swiglu(x64[t:t + 1], _decode_np(gu_p[e], gu_s[e], tab),
                                 _decode_np(dn_p[e], dn_s[e], tab), F)
            ref[t] += float(w[t, j]) * y[0]
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 5e-3


def test_moe_token_subset_and_expert_identity(golden_dir):
    """Computing a subset of tokens gives the same rows; swapping two experts' weights together
    with the routing indices leaves the output unchanged (catches expert-offset mistakes)."""
    T, H, F, E, k = 7, 64, 32, 4, 2
    x, gu_p, gu_s, dn_p, dn_s = _small_moe(18, T, H, F, E, k)
    r = np.random.default_rng(18)
    idx = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = r.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    full = oracle.moe_mlp(x, idx, w, gu_p, gu_s, dn_p, dn_s, E=E)
    sub = oracle.moe_mlp(x, idx, w, gu_p, gu_s, dn_p, dn_s, E=E, tokens=[5, 0, 3])
    np.testing.assert_array_equal(sub, full[[5, 0, 3]])
    sw = np.array([1, 0, 2, 3])
    idx2 = sw[idx].astype(np.int32)
    out2 = oracle.moe_mlp(x, idx2, w, gu_p[sw], gu_s[sw], dn_p[sw], dn_s[sw], E=E)
    np.testing.assert_array_equal(out2, full)
    # the routing weight scales the expert output linearly
    out3 = oracle.moe_mlp(x, idx, w * 2, gu_p, gu_s, dn_p, dn_s, E=E)
    np.testing.assert_allclose(out3, 2 * full, rtol=1e-12, atol=1e-300)


def test_moe_mx_act_quantizes_both_activations(golden_dir):
    """Activation variant, E = k = 1: x and the bf16 h are quantized along their rows."""
    tab = _table(golden_dir)
    T, H, F = 4, 64, 96
    x, gu_p, gu_s, dn_p, dn_s = _small_moe(19, T, H, F, 1, 1)
    idx = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    out, h = oracle.moe_mlp(x, idx, w, gu_p, gu_s, dn_p, dn_s, E=1, mx_act=True, want_h=True)
    xq = _decode_np(*oracle.quantize(x), tab)
    a = xq @ _decode_np(gu_p[0], gu_s[0], tab).T
    g, u = a[:, :F], a[:, F:]
    href = _bf16_round(g / (1 + np.exp(-g)) * u)
    hgot = _bf16_f64(h[:, 0, :])
    np.testing.assert_allclose(hgot, href, rtol=2 ** -7, atol=1e-30)
    hq = _decode_np(*oracle.quantize(h[:, 0, :].copy()), tab)
    ref = hq @ _decode_np(dn_p[0], dn_s[0], tab).T
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-14)
