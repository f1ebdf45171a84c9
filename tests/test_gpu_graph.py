"""GPU: the whole MoE MLP recorded once into a HIP graph and replayed.

mxfp4_moe_mlp enqueues kernels only (no allocation, memset, copy or synchronization), so a caller
can capture it on a stream. Each replay must reproduce the eager call bit for bit; between
replays the test does eager work on the same buffers (clearing the output with a fill kernel,
writing new activations) and checks that the next replay reads the buffers as they are then."""
import numpy as np
import pytest
import torch

from mxfp4_weight_quantized_amd import inputs
import mxfp4_weight_quantized_amd as mx
from parity_util import moe_weights_dev, note, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="held back: its only GPU run died in the HIP runtime's first-use "
                            "initialisation (segmentation fault inside torch.cuda lazy init, "
                            "before any graph code ran, in a process whose first GPU use came "
                            "after multi-threaded oracle packing); no cause shown yet (the oracle "
                            "is clean under AddressSanitizer), so the case stays off the GPU"),
]


def _tiled(wdev):
    gp, gs, dp, ds = wdev
    return (*mx.mxfp4_tile_weights(gp, gs), *mx.mxfp4_tile_weights(dp, ds))


@pytest.mark.parametrize("T,H,F,E,k,flags,tiled", [
    (1, 256, 192, 16, 4, 0, True),               # decode-shaped, a single token
    (64, 256, 192, 8, 2, 0, False),              # decode-shaped, row-major weights
    (600, 128, 96, 4, 2, 0, True),               # prefill-shaped tiles
    (300, 128, 128, 8, 4, mx.MX_ACT_MXFP4, True),  # activation variant
])
def test_moe_mlp_replays_in_a_graph(T, H, F, E, k, flags, tiled):
    seed = 500 + T
    wd = moe_weights_dev(seed, E, H, F)
    w = _tiled(wd) if tiled else wd
    fl = flags | (mx.MX_WEIGHTS_TILED if tiled else 0)
    wr, br = inputs.router(seed, E, H, 0.5)
    wr_d, br_d = to_dev(wr), to_dev(br)
    x_static = to_dev(inputs.activations(seed, T, H))
    x_next = to_dev(inputs.activations(seed + 1, T, H))
    out_g = torch.empty((T, H), dtype=torch.float32, device="cuda")
    desc = mx.make_moe_desc(x_static, *w, k, out_g, wr=wr_d, br=br_d, flags=fl)
    ws = torch.empty(mx.mxfp4_moe_mlp_workspace(desc), dtype=torch.uint8, device="cuda")

    def eager(x):
        return mx.mxfp4_moe_mlp(x, *w, k, wr=wr_d, br=br_d, out_dtype=torch.float32, flags=fl)

    note("graph replay T=%d H=%d F=%d E=%d k=%d flags=%d" % (T, H, F, E, k, fl))
    ref0 = eager(x_static)
    ref1 = eager(x_next)
    # warm the path on the capture buffers, then capture one call
    mx.mxfp4_moe_mlp(x_static, *w, k, wr=wr_d, br=br_d, flags=fl, out=out_g, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mx.mxfp4_moe_mlp(x_static, *w, k, wr=wr_d, br=br_d, flags=fl, out=out_g, workspace=ws)
    torch.cuda.synchronize()
    x0 = x_static.clone()
    for rep in range(4):
        src = x0 if rep % 2 == 0 else x_next
        x_static.copy_(src)   # eager work on the graph's input
        out_g.zero_()         # and on its output (a fill kernel)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref0 if rep % 2 == 0 else ref1), "replay %d" % rep
    # the eager path still works with the same workspace after the replays
    again = eager(x0)
    torch.cuda.synchronize()
    assert torch.equal(again, ref0)
    assert np.isfinite(out_g.cpu().numpy()).all()
