"""GPU: mxfp4_moe_mlp_noalloc, whose workspace is the library's own device array, against
mxfp4_moe_mlp with a caller workspace, through the C ABI. Two calls in a row, the second with a
smaller input (the array keeps the first call's contents), each equal bit for bit to the
workspace entry point on the same inputs (the same kernels and arithmetic). (The rejection of
problems beyond the array is a host check, tested without a GPU in test_abi_host.py.)"""
import ctypes

import numpy as np
import pytest
import torch

from mxfp4_weight_quantized_amd import inputs
import mxfp4_weight_quantized_amd as mx
from parity_util import layer_weights_dev, note, tiled_dev, to_dev

pytestmark = pytest.mark.gpu


def _pair(x, wts, wr, br, k, flags, out_dtype):
    """(workspace entry point's output, allocation-free entry point's output) on one input."""
    T, H = x.shape
    outs = []
    for noalloc in (False, True):
        out = torch.empty((T, H), dtype=out_dtype, device="cuda")
        d = mx.make_moe_desc(x, *wts, k, out, wr=wr, br=br, flags=flags)
        if noalloc:
            assert mx.mxfp4_moe_mlp_workspace(d) <= mx.MX_NOALLOC_SCRATCH_BYTES
            mx.mxfp4_moe_mlp_noalloc(d)
        else:
            ws = torch.empty(mx.mxfp4_moe_mlp_workspace(d), dtype=torch.uint8, device="cuda")
            mx._check(mx.lib().mxfp4_moe_mlp(ctypes.byref(d), ws.data_ptr(), ws.numel(),
                                             mx._stream(None)))
        torch.cuda.synchronize()
        outs.append(out)
    return outs


@pytest.mark.parametrize("flags", [mx.MX_WEIGHTS_TILED, mx.MX_WEIGHTS_TILED | mx.MX_ACT_MXFP4])
def test_noalloc_equals_workspace_entry_point(flags):
    s = inputs.MOE_20B_DECODE  # T = 64, H = F = 2880, E = 32, top-4
    wts = tiled_dev(layer_weights_dev(s.seed, s.E, s.H, s.F))
    wr, _ = inputs.router(s.seed, s.E, s.H, 0.0)
    wr = to_dev(wr)
    x = to_dev(inputs.activations(s.seed, s.T, s.H))
    note("noalloc call 1: T=%d flags=%d" % (s.T, flags))
    a, b = _pair(x, wts, wr, None, s.k, flags, torch.float32)
    assert torch.equal(a, b)
    assert torch.isfinite(a).all() and a.abs().max() > 0
    # second call, smaller input, other tokens (the array still holds the first call's rows)
    x2 = to_dev(inputs.activations(s.seed + 1, 5, s.H))
    note("noalloc call 2: T=5 flags=%d" % flags)
    a2, b2 = _pair(x2, wts, wr, None, s.k, flags, torch.bfloat16)
    assert torch.equal(a2, b2)
    assert mx.get_device_error() == 0
