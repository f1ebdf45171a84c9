"""GPU parity of the MXFP4 codec (mxfp4_quantize / mxfp4_dequantize): bit-exact with the oracle."""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_weight_quantized_amd import inputs
import mxfp4_weight_quantized_amd as mx
from parity_util import DEV, bf16_host_bits, note, to_dev

pytestmark = pytest.mark.gpu


def _gpu_quantize(x_np):
    t = to_dev(x_np)
    p, s = mx.mxfp4_quantize(t)
    torch.cuda.synchronize()
    return p.cpu().numpy(), s.cpu().numpy()


def _special_blocks():
    """Blocks over the whole fp32 range: every binade, ties, saturation, zeros, subnormals,
    the clamp region, NaN and Inf."""
    r = np.random.default_rng(100)
    blocks = []
    for e in range(-149, 128, 3):  # amax in every third binade, including subnormals
        b = r.uniform(-1, 1, 32) * 2.0 ** e
        blocks.append(b)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.99, 4.0, 0.0])
    for sc in (-130, -126, -100, 0, 17, 120):
        b = r.choice(mids, 32) * r.choice([-1, 1], 32)
        b[0] = 4.0
        blocks.append(b * 2.0 ** sc)
    blocks.append(np.zeros(32))
    blocks.append(-np.zeros(32))
    z = np.zeros(32); z[3] = np.nan; blocks.append(z)
    z = np.ones(32); z[31] = -np.inf; blocks.append(z)
    z = np.ones(32); z[0] = np.inf; blocks.append(z)
    z = np.full(32, 1e-45); blocks.append(z)                         # smallest subnormal
    z = np.full(32, 2.0 ** -127); z[1] = -3 * 2.0 ** -129; blocks.append(z)
    z = np.full(32, 3.4e38); blocks.append(z)                        # near the fp32 max
    return np.array(blocks, np.float64).astype(np.float32)


def test_quantize_f32_special_blocks_bit_exact():
    x = _special_blocks()
    note("quantize f32 special blocks %s" % (x.shape,))
    gp, gs = _gpu_quantize(x)
    op, os_ = oracle.quantize(x)
    np.testing.assert_array_equal(gs, os_)
    np.testing.assert_array_equal(gp, op)


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 64), (7, 96), (64, 2880), (5760, 2880)])
def test_quantize_f32_weights_bit_exact(rows, K):
    x = inputs.normal_f32(21, inputs.TAG_MISC, (rows, K), 0.02, sub=rows)
    x[0, :7] = [0.0, -0.0, 1e-40, 0.25 * 2 ** -6, 7.9, -5.0, 3.5]  # odd values in the first block
    note("quantize f32 %dx%d" % (rows, K))
    gp, gs = _gpu_quantize(x)
    op, os_ = oracle.quantize(x)
    np.testing.assert_array_equal(gs, os_)
    np.testing.assert_array_equal(gp, op)


def test_quantize_bf16_all_bit_patterns():
    """All 65536 bf16 patterns (NaNs and Infs included) as 2048 blocks."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(2048, 32)
    note("quantize bf16 all patterns")
    gp, gs = _gpu_quantize(bits)
    op, os_ = oracle.quantize(bits)
    np.testing.assert_array_equal(gs, os_)
    np.testing.assert_array_equal(gp, op)
    # and a shuffled arrangement so that finite blocks mix small and large values
    r = np.random.default_rng(22)
    sh = bits.reshape(-1)[r.permutation(65536)].reshape(2048, 32)
    gp, gs = _gpu_quantize(sh)
    op, os_ = oracle.quantize(sh)
    np.testing.assert_array_equal(gs, os_)
    np.testing.assert_array_equal(gp, op)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_exhaustive(dtype):
    """Every code (16) under every scale byte (256), both output types."""
    packed = np.zeros((256, 16), np.uint8)
    for j in range(16):
        packed[:, j] = ((2 * j) % 16) | (((2 * j + 1) % 16) << 4)
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    note("dequantize exhaustive %s" % dtype)
    out = mx.mxfp4_dequantize(to_dev(packed), to_dev(scales), dtype=dtype)
    torch.cuda.synchronize()
    ref = oracle.dequantize(packed, scales)
    if dtype == torch.float32:
        got = out.cpu().numpy()
        want = ref.astype(np.float32)
        np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
        ok = ~np.isnan(want)
        np.testing.assert_array_equal(got.view(np.uint32)[ok], want.view(np.uint32)[ok])
    else:
        got = bf16_host_bits(out)
        want = np.array([oracle.bf16_from_double(v) for v in ref.reshape(-1)], np.uint16).reshape(ref.shape)
        nan = np.isnan(ref)
        np.testing.assert_array_equal(got[~nan], want[~nan])
        assert np.all((got[nan] & 0x7f80) == 0x7f80) and np.all((got[nan] & 0x7f) != 0)


def test_dequantize_roundtrip_full_weight():
    x = inputs.gate_up_f32(2, 0, 2880, 2880)
    op, os_ = oracle.quantize(x)
    note("dequantize 5760x2880")
    out = mx.mxfp4_dequantize(to_dev(op), to_dev(os_), dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.dequantize(op, os_).astype(np.float32)
    np.testing.assert_array_equal(out.cpu().numpy(), ref)


def test_quantize_empty_is_noop():
    t = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    p, s = mx.mxfp4_quantize(t)
    assert p.shape == (0, 32) and s.shape == (0, 2)
