"""Pins for the oracle's MXFP4 codec (CPU only).

Each test checks the oracle against something other than itself: the hand-written value table
and hand-worked blocks under tests/golden/, closed forms (powers of two), invariants of the scale
rule, and an independent formulation of the rounding (generic round-half-even to a float grid).
"""
import math
import os

import numpy as np
import pytest

import oracle

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _load_table(golden_dir):
    tab = {}
    with open(os.path.join(golden_dir, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            tab[int(c, 16)] = float(v)
    return tab


def _load_blocks(golden_dir):
    blocks, cur = [], None
    with open(os.path.join(golden_dir, "quant_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            if key == "block":
                cur = {"name": rest[0]}
                blocks.append(cur)
            elif key == "in":
                cur["in"] = [float(v) for v in rest]
            elif key == "scale":
                cur["scale"] = int(rest[0])
            elif key == "packed":
                cur["packed"] = [int(v, 16) for v in rest]
    return blocks


def test_e2m1_table_matches_golden(golden_dir):
    tab = _load_table(golden_dir)
    assert sorted(tab) == list(range(16))
    for c, v in tab.items():
        got = oracle.e2m1_value(c)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), (c, got, v)


def test_e8m0_closed_form():
    for b in range(255):
        assert oracle.e8m0_value(b) == 2.0 ** (b - 127), b
    assert math.isnan(oracle.e8m0_value(255))


def test_dequantize_exhaustive_codes_and_scales(golden_dir):
    """All 16 codes x 256 scale bytes: value = table[code] * 2^(b-127) (NaN for b = 255)."""
    tab = _load_table(golden_dir)
    R = 256
    packed = np.zeros((R, 16), np.uint8)
    for j in range(16):  # element 2j = code (2j % 16), element 2j+1 = code (2j+1) % 16
        packed[:, j] = ((2 * j) % 16) | (((2 * j + 1) % 16) << 4)
    scales = np.arange(256, dtype=np.uint8).reshape(R, 1)
    out = oracle.dequantize(packed, scales)
    for b in range(256):
        for i in range(32):
            exp = tab[i % 16] * 2.0 ** (b - 127) if b < 255 else float("nan")
            got = out[b, i]
            if b == 255:
                assert math.isnan(got)
            else:
                assert got == exp and math.copysign(1, got) == math.copysign(1, exp), (b, i)


def test_golden_blocks(golden_dir):
    blocks = _load_blocks(golden_dir)
    assert len(blocks) >= 8
    for blk in blocks:
        x = np.zeros((1, 32), np.float32)
        x[0, :len(blk["in"])] = np.array(blk["in"], np.float32)
        p, s = oracle.quantize(x)
        assert int(s[0, 0]) == blk["scale"], blk["name"]
        assert [int(v) for v in p[0]] == blk["packed"], (blk["name"], [hex(v) for v in p[0]])


def _random_blocks(n, seed):
    """Blocks whose magnitudes spread over many binades, with some exact grid points mixed in."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((n, 32)).astype(np.float32)
    x *= np.float32(2.0) ** r.integers(-60, 60, size=(n, 1)).astype(np.float32)
    # sprinkle exact ties / grid values (relative to a block scale of 2^0 after the rule below)
    return x


def _independent_round(a):
    """E2M1 magnitude by generic float rounding: spacing 0.5 below 2, 1 in [2, 4), 2 in [4, 8);
    numpy's round is round-half-even on the quotient; results above 6 clamp to 6."""
    spacing = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    return np.minimum(np.round(a / spacing) * spacing, 6.0)


def test_scale_rule_brackets_amax():
    """For every non-clamped block: 2^(s+2) <= amax < 2^(s+3), s = byte - 127 (comparisons only)."""
    x = _random_blocks(4000, 1)
    p, s = oracle.quantize(x)
    amax = np.abs(x.astype(np.float64)).max(axis=1)
    sb = s[:, 0].astype(np.int64) - 127
    lo = np.array([2.0 ** int(v + 2) for v in sb])
    assert np.all(sb > -127)
    assert np.all(lo <= amax) and np.all(amax < 2 * lo)


def test_codes_match_independent_rounding():
    x = _random_blocks(4000, 2)
    # add blocks that hit the tie points exactly: grid midpoints times a power of two
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 6.5, 7.99], np.float32)
    r = np.random.default_rng(3)
    ties = r.choice(mids, size=(2000, 32)).astype(np.float32) * r.choice([-1, 1], size=(2000, 32))
    ties[:, 0] = 4.0  # pins the block scale to 2^0 so the mids stay exact ties
    ties *= np.float32(2.0) ** r.integers(-20, 20, size=(2000, 1)).astype(np.float32)
    x = np.concatenate([x, ties.astype(np.float32)])
    p, s = oracle.quantize(x)
    vals = oracle.dequantize(p, s)
    scale = 2.0 ** (s[:, 0].astype(np.float64) - 127)
    a = np.abs(x.astype(np.float64)) / scale[:, None]
    expect = _independent_round(a) * np.where(np.signbit(x), -1.0, 1.0) * scale[:, None]
    np.testing.assert_array_equal(vals, expect)
    # the sign bit follows the input's sign bit even when the value rounds to zero
    codes = np.stack([p & 15, p >> 4], axis=-1).reshape(x.shape)
    np.testing.assert_array_equal((codes >> 3).astype(bool), np.signbit(x))


def test_roundtrip_of_representable_blocks():
    """Blocks built from grid values times 2^s whose largest magnitude is 4 or 6 reproduce their
    codes and scale byte exactly."""
    r = np.random.default_rng(4)
    for trial in range(500):
        s = int(r.integers(-120, 120))
        codes = r.integers(0, 16, size=32)
        top = int(r.choice([6, 7]))
        codes[r.integers(0, 32)] = top | (int(r.integers(0, 2)) << 3)
        codes = np.where((codes & 7) > top, (codes & 8) | top, codes)
        vals = np.array([(-1.0 if c & 8 else 1.0) * GRID[c & 7] for c in codes]) * 2.0 ** s
        x = vals.astype(np.float32).reshape(1, 32)
        p, sc = oracle.quantize(x)
        assert int(sc[0, 0]) == s + 127
        got = np.stack([p[0] & 15, p[0] >> 4], axis=-1).reshape(32)
        np.testing.assert_array_equal(got, codes)


def test_idempotent_values():
    """quantize(dequantize(q)) has the same values as q (unclamped scales)."""
    r = np.random.default_rng(5)
    p = r.integers(0, 256, size=(300, 16)).astype(np.uint8)
    s = r.integers(20, 230, size=(300, 1)).astype(np.uint8)
    v = oracle.dequantize(p, s)
    p2, s2 = oracle.quantize(v.astype(np.float32))
    v2 = oracle.dequantize(p2, s2)
    nz = np.abs(v).max(axis=1) > 0
    np.testing.assert_array_equal(v2[nz], v[nz])


def test_monotone_at_fixed_scale():
    r = np.random.default_rng(6)
    base = np.sort(r.uniform(-7.9, 7.9, size=(200, 31)), axis=1).astype(np.float32)
    x = np.concatenate([base, np.full((200, 1), 7.95, np.float32)], axis=1)  # amax fixes s = 0
    p, s = oracle.quantize(x)
    assert np.all(s == 127)
    v = oracle.dequantize(p, s)[:, :31]
    assert np.all(np.diff(v, axis=1) >= 0)


def test_bf16_input_equals_widened_f32_input():
    r = np.random.default_rng(7)
    x = (r.standard_normal((64, 96)) * 3).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern will do
    xw = (xb.astype(np.uint32) << 16).view(np.float32)
    pa, sa = oracle.quantize(xb)
    pb, sb = oracle.quantize(xw)
    np.testing.assert_array_equal(pa, pb)
    np.testing.assert_array_equal(sa, sb)


def test_storage_ratio_about_four():
    """17/32 bytes per weight vs 2 for bf16: the roughly fourfold saving the English page's
    "Native Support" and "Memory Savings" passages describe."""
    K, R = 2880, 8
    p, s = oracle.quantize(np.ones((R, K), np.float32))
    ratio = (R * K * 2) / (p.nbytes + s.nbytes)
    assert abs(ratio - 64 / 17) < 1e-12 and 3.5 < ratio < 4.0


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(8)
    f = np.concatenate([
        (r.standard_normal(20000) * 10.0 ** r.integers(-30, 30, 20000)).astype(np.float32),
        # exact ties: 8 significant bits plus a half ulp
        ((np.arange(1, 2000, dtype=np.float32) * 2 + 1) * np.float32(2.0 ** -9)),
        np.array([1e-40, -3e-39, 3.3895e38, -0.0, 0.0], np.float32),
    ])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_double(float(v)) for v in f], np.uint16)
    np.testing.assert_array_equal(got, want)
