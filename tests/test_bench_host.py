"""CPU: the benchmark's own accounting (no GPU).

The bench line's roofline divides a kernel's algorithmic flops or bytes by its measured time; these
tests pin those work figures to closed forms of the MXFP4 layout (a packed weight costs half a
byte for its E2M1 code plus 1/32 byte for its share of the block's E8M0 scale: 17/32 byte) and to
the workload shapes, and check the bound chosen for each regime and the single-GPU refusal."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from mxfp4_weight_quantized_amd import inputs  # noqa: E402


def test_packed_layer_bytes_match_the_format():
    # 20B-shaped layer: 32 experts, gate_up [5760 x 2880] and down [2880 x 2880] per expert,
    # 4 bits per weight plus one scale byte per 32 weights
    s = inputs.MOE_20B_DECODE
    weights = s.E * (2 * s.F * s.H + s.H * s.F)
    packed = weights // 2 + weights // 32
    assert packed == 423_014_400
    gu_flops, gu_bytes = bench.kernel_work("moe_gate_up_swiglu", s.T, s.H, s.F, s.E, s.k,
                                           touched=s.E, P=s.T * s.k, out_bytes=2, mxact=False)
    dn_flops, dn_bytes = bench.kernel_work("moe_down_weighted", s.T, s.H, s.F, s.E, s.k,
                                           touched=s.E, P=s.T * s.k, out_bytes=2, mxact=False)
    P = s.T * s.k
    # weight bytes of both products = the packed layer; activations: x in, h out, h in, y out
    assert gu_bytes + dn_bytes == packed + s.T * s.H * 2 + P * s.F * 2 + P * s.F * 2 + P * s.H * 4
    assert gu_flops == 2 * P * s.H * 2 * s.F and dn_flops == 2 * P * s.F * s.H


def test_prefill_flops_and_activation_variant_bytes():
    s = inputs.MOE_20B_PREFILL
    P = s.T * s.k
    fl_gu, by_gu = bench.kernel_work("moe_gate_up_swiglu", s.T, s.H, s.F, s.E, s.k, s.E, P, 2, False)
    fl_dn, _ = bench.kernel_work("moe_down_weighted", s.T, s.H, s.F, s.E, s.k, s.E, P, 2, False)
    assert fl_gu + fl_dn == pytest.approx(1.6307e12, rel=1e-4)  # 3 products of 2*P*H*F flops
    # with MXFP4 activations x and h cost 17/32 byte per element instead of 2
    _, by4 = bench.kernel_work("moe_gate_up_swiglu", s.T, s.H, s.F, s.E, s.k, s.E, P, 2, True)
    assert by_gu - by4 == pytest.approx((s.T * s.H + P * s.F) * (2 - 17 / 32))


def test_roofline_bound_follows_the_ridge():
    # bf16 ridge: 2500 TFLOP/s over 8 TB/s = 312.5 flop per byte
    pre = bench.roofline_entry(1e12, 1e9, 1.0, bench.PEAK_BF16_TFLOPS)
    assert pre["bound"] == "mfma" and pre["achieved"] == pytest.approx(1000.0)
    assert pre["frac"] == pytest.approx(0.4)
    dec = bench.roofline_entry(1e9, 4e8, 0.1, bench.PEAK_BF16_TFLOPS)
    assert dec["bound"] == "hbm" and dec["achieved"] == pytest.approx(4000.0)
    assert dec["frac"] == pytest.approx(0.5)


def test_workload_names_cover_the_configurations():
    wl = bench.workloads()
    assert bench.DEFAULT_WORKLOAD in wl and bench.DECODE_WORKLOAD in wl
    for name in ("moe-20b-decode-T64", "moe-20b-prefill-T8192-skewed", "moe-120b-T1",
                 "moe-120b-T256", "moe-120b-T4096", "moe-120b-mxact-T4096",
                 "linear-decode-M1", "linear-decode-M8", "linear-decode-M32"):
        assert name in wl


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
