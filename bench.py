#!/usr/bin/env python3
"""Benchmark of the MXFP4 weight-quantized MoE-MLP hot path on one MI355X.

One step = one ``mxfp4_moe_mlp`` call (router -> permutation -> gate_up grouped GEMM with SwiGLU
-> down grouped GEMM -> combine) over one batch of synthetic tokens, inputs resident in HBM.
Prints ONE JSON line: tokens/s for the whole step, plus the roofline of the dominant kernel
(timed with HIP events recorded by the library on the stream it launches on) and the CPU oracle
timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME]
  python bench.py --summarize-counters DIR_FETCH DIR_WRITE   (rocprofv3 --pmc output -> profiles/)

Decode-shaped workloads rotate through several copies of the weights (and several token
batches) so the working set exceeds the 256 MB Infinity Cache and every step reads HBM.

The default run (the prefill layer) also times the 20B-shaped decode layer (T = 64) in the same
process and adds it to the line as ``decode`` (the metric's decode HBM GB/s half); --no-decode
leaves it out.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "mxfp4_weight_quantized_amd", "csrc", "gemm.hip")

METRIC = "MXFP4 MoE-MLP tokens/s; decode HBM GB/s; prefill TFLOP/s vs peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP4_TFLOPS = 10100.0      # dense fp4 MFMA
CACHE_BYTES = 256 << 20        # Infinity Cache (MALL)
DEFAULT_WORKLOAD = "moe-20b-prefill-T8192-skewed"


def workloads():
    from mxfp4_weight_quantized_amd import inputs
    w = {}
    for s in (inputs.MOE_20B_DECODE, inputs.MOE_20B_PREFILL, *inputs.MOE_120B.values()):
        w[s.name] = ("moe", s, 0)
    for T in (1, 256, 4096):
        s = inputs.MOE_120B[T]
        w["moe-120b-mxact-T%d" % T] = ("moe", s, 1)
    w[inputs.MOE_20B_PREFILL.name + "-mxact"] = ("moe", inputs.MOE_20B_PREFILL, 1)
    w[inputs.MOE_20B_DECODE.name + "-mxact"] = ("moe", inputs.MOE_20B_DECODE, 1)
    # decode-shaped layers as one launch (MX_SINGLE_LAUNCH = 0x4)
    for s in (inputs.MOE_20B_DECODE, inputs.MOE_120B[1], inputs.MOE_120B[256]):
        w[s.name + "-single"] = ("moe", s, 4)
    for M in (1, 8, 32):
        w["linear-decode-M%d" % M] = ("linear", dict(M=M, K=2880, N=5760, seed=1), 0)
    return w


def source_sha() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "mxfp4_weight_quantized_amd", "csrc", "*"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------------------------
def _upload_bf16(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def setup_moe(shape, flags, want_host_weights):
    """Device inputs for a MoE layer; weights drawn in fp32 and packed by the HIP quantizer.
    With want_host_weights the same draws are also packed by the oracle for the CPU leg."""
    import numpy as np
    import torch
    import mxfp4_weight_quantized_amd as mx
    from mxfp4_weight_quantized_amd import inputs
    s = shape
    E, H, F = s.E, s.H, s.F
    gp = torch.empty((E, 2 * F, H // 2), dtype=torch.uint8, device="cuda")
    gs = torch.empty((E, 2 * F, H // 32), dtype=torch.uint8, device="cuda")
    dp = torch.empty((E, H, F // 2), dtype=torch.uint8, device="cuda")
    ds = torch.empty((E, H, F // 32), dtype=torch.uint8, device="cuda")
    host = None
    if want_host_weights:
        host = [np.empty(t.shape, np.uint8) for t in (gp, gs, dp, ds)]
        import oracle

    def draw(e):
        return e, inputs.gate_up_f32(s.seed, e, F, H), inputs.down_f32(s.seed, e, H, F)

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(8) as ex:
        for e, wgu, wdn in ex.map(draw, range(E)):
            mx.mxfp4_quantize(torch.from_numpy(wgu).cuda(), gp[e], gs[e])
            mx.mxfp4_quantize(torch.from_numpy(wdn).cuda(), dp[e], ds[e])
            if host is not None:
                host[0][e], host[1][e] = oracle.quantize(wgu)
                host[2][e], host[3][e] = oracle.quantize(wdn)
    torch.cuda.synchronize()
    wr, br = inputs.router(s.seed, E, H, s.bias_std)
    return (gp, gs, dp, ds), wr, (br if s.bias_std else None), host


def touched_stats(idx_np, E):
    import numpy as np
    cnt = np.bincount(idx_np.reshape(-1), minlength=E)
    return int((cnt > 0).sum()), int(cnt.sum())


def kernel_work(name, T, H, F, E, k, touched, P, out_bytes, mxact):
    """Algorithmic (flops, bytes) of one launch of a kernel kind."""
    wb = 17.0 / 32.0                 # packed bytes per weight (nibble + 1/32 scale byte)
    abytes = 17.0 / 32.0 if mxact else 2.0   # activation bytes per element read by a GEMM
    if name == "moe_gate_up_swiglu":   # h out: bf16, or MXFP4 (quantized in the epilogue)
        return 2.0 * P * H * 2 * F, touched * 2 * F * H * wb + T * H * abytes + P * F * abytes
    if name == "moe_down_weighted":
        return 2.0 * P * F * H, touched * H * F * wb + P * F * abytes + P * H * 4
    if name == "moe_combine":
        return P * H, P * H * 4 + T * H * out_bytes
    if name == "route_topk":
        return 2.0 * T * E * H, T * H * 2 + E * H * 2 + T * E * 4 + T * k * 8
    if name == "permute":
        return 0.0, T * k * 4 * 4 + (E + 1) * 4
    if name == "moe_single_launch":  # the whole layer: its touched weights, x, W_r, out
        return (2.0 * P * 3 * F * H + 2.0 * T * E * H,
                touched * 3 * F * H * wb + T * H * 2 + E * H * 2 + T * H * out_bytes)
    if name == "quantize":   # activation variant: x along H (h is quantized by gate_up)
        return 0.0, T * H * (2 + wb)
    return 0.0, 0.0


def roofline_entry(flops, nbytes, avg_ms, peak_mfma):
    ridge = peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9)
    if nbytes > 0 and flops / nbytes > ridge:
        ach = flops / (avg_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_mfma,
                "unit": "TFLOP/s", "frac": round(ach / peak_mfma, 4)}
    ach = nbytes / (avg_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4)}


def read_traffic(workload, kernel):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were taken on the
    current kernel sources; else None."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = data.get(workload, {}).get(kernel)
    if not ent or ent.get("source_sha") != source_sha():
        return None
    return ent.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------------------------
def bench_moe(args, name, shape, flags):
    import numpy as np
    import torch
    import mxfp4_weight_quantized_amd as mx
    from mxfp4_weight_quantized_amd import inputs
    s = shape
    want_cpu = not args.no_cpu_baseline
    weights, wr_np, br_np, host_w = setup_moe(s, flags, want_cpu)
    tiled = not args.row_major_weights
    if tiled:  # the kernels' weight layout, converted once (weights are static)
        gp, gs, dp, ds = weights
        weights = (*mx.mxfp4_tile_weights(gp, gs), *mx.mxfp4_tile_weights(dp, ds))
        del gp, gs, dp, ds
        torch.cuda.synchronize()
    desc_flags = flags | (mx.MX_WEIGHTS_TILED if tiled else 0)
    wr = _upload_bf16(wr_np)
    br = torch.from_numpy(br_np).cuda() if br_np is not None else None
    layer_bytes = s.E * (2 * s.F * s.H + s.H * s.F) * 17 // 32
    # token batches: decode-shaped runs rotate through several batches (different experts)
    n_x = 1 if s.T * s.k >= 48 * s.E else 16
    x_all = inputs.activations(s.seed, s.T * n_x, s.H)
    xs = [_upload_bf16(x_all[i * s.T:(i + 1) * s.T]) for i in range(n_x)]
    # routing of every batch (outside the timed region) -> touched experts per step
    stats = []
    for x in xs:
        _, idx, _ = mx.moe_route_topk(x, wr, br, s.k, want_logits=False)
        stats.append(touched_stats(idx.cpu().numpy(), s.E))
    touched = float(np.mean([t for t, _ in stats]))
    step_bytes = touched * layer_bytes / s.E
    n_w = 1
    if step_bytes * n_x < 2 * CACHE_BYTES or layer_bytes < 2 * CACHE_BYTES:
        n_w = int(min(8, max(1, math.ceil(2 * CACHE_BYTES / max(1.0, min(layer_bytes, step_bytes * n_x))))))
    wsets = [weights] + [tuple(t.clone() for t in weights) for _ in range(n_w - 1)]
    out_dtype = torch.bfloat16
    out = torch.empty((s.T, s.H), dtype=out_dtype, device="cuda")
    descs = []
    for i in range(max(n_x, n_w)):
        gp, gs, dp, ds = wsets[i % n_w]
        descs.append(mx.make_moe_desc(xs[i % n_x], gp, gs, dp, ds, s.k, out, wr=wr, br=br,
                                      flags=desc_flags))
    ws_bytes = max(mx.mxfp4_moe_mlp_workspace(d) for d in descs)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    L = mx.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    import ctypes
    refs = [ctypes.byref(d) for d in descs]

    def step(i):
        st = L.mxfp4_moe_mlp(refs[i % len(refs)], ws.data_ptr(), ws_bytes, sh)
        if st != 0:
            raise mx.MXError(st, mx.last_error())

    settle = settle_clocks(step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    if args.graph:
        # one HIP graph holds one rotation of the step over the token batches / weight copies;
        # the timed steps are whole rotations (steps rounded up to a multiple of the period)
        period = len(refs)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream().cuda_stream
            for i in range(period):
                st = L.mxfp4_moe_mlp(refs[i], ws.data_ptr(), ws_bytes, cap)
                if st != 0:
                    raise mx.MXError(st, mx.last_error())
        reps = max(1, -(-args.steps // period))
        g.replay()
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(reps):
            g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        timed_steps = reps * period
    else:
        t0.record(stream)
        for i in range(args.steps):
            step(i)
        t1.record(stream)
        torch.cuda.synchronize()
        timed_steps = args.steps
    ms = t0.elapsed_time(t1) / timed_steps

    # per-kernel times over a second pass of the same steps (events recorded by the library)
    mx.mx_profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    prof = mx.mx_profile_read()
    mx.mx_profile_enable(False)

    P = s.T * s.k
    mxact = bool(flags & 1)  # MX_ACT_MXFP4
    peak = PEAK_FP4_TFLOPS if mxact else PEAK_BF16_TFLOPS
    kern = {}
    for kname, (n, tot) in prof.items():
        fl, by = kernel_work(kname, s.T, s.H, s.F, s.E, s.k, touched, P, 2, mxact)
        kern[kname] = {"avg_ms": round(tot / n, 5), "launches": n, "flops": fl, "bytes": by}
    dom = max(kern, key=lambda k: kern[k]["avg_ms"] * kern[k]["launches"])
    d = kern[dom]
    roof = roofline_entry(d["flops"], d["bytes"], d["avg_ms"], peak)
    roof["traffic"] = read_traffic(name, dom)
    roof["kernel"] = dom
    roof["avg_ms"] = d["avg_ms"]
    roof["algorithmic_bytes"] = int(d["bytes"])
    roof["algorithmic_flops"] = d["flops"]

    layer_flops = 2.0 * P * (s.H * 2 * s.F + s.F * s.H)
    layer_traffic = touched * layer_bytes / s.E + s.T * s.H * 2 * 2
    result = {
        "metric": METRIC, "value": round(s.T / (ms * 1e-3), 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": timed_steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4" if mxact else "bf16", "data": "synthetic",
        "config": {"workload": name, "T": s.T, "H": s.H, "F": s.F, "E": s.E, "k": s.k,
                   "weights": "mxfp4 (e2m1 + e8m0 per 32)",
                   "weight_layout": "tiled (converted once at load)" if tiled else "row-major",
                   "activations": "mxfp4" if mxact else "bf16",
                   "out_dtype": "bf16", "router_bias_std": s.bias_std, "seed": s.seed,
                   "parallelism": "single-gpu", "weight_copies": n_w, "token_batches": n_x,
                   "launch": ("one persistent kernel per step" if flags & 4 else
                              "hip graph per rotation" if args.graph else "eager")},
        "settle": settle,
        # the whole call against the same roofline as the dominant kernel (whose figure
        # "roofline" is kernel-level): MFMA peak for prefill-shaped layers, HBM for decode-shaped
        "step": {"tflops": round(layer_flops / (ms * 1e-3) / 1e12, 2),
                 "hbm_gbs_algorithmic": round(layer_traffic / (ms * 1e-3) / 1e9, 1),
                 "touched_experts": touched,
                 "bound": roof["bound"],
                 "frac": round(layer_flops / (ms * 1e-3) / 1e12 / peak if roof["bound"] == "mfma"
                               else layer_traffic / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "kernels": kern,
        "roofline": roof,
    }
    if want_cpu:
        result["cpu_baseline"] = cpu_baseline_moe(args, s, x_all[:s.T], wr_np, br_np, host_w,
                                                  mxact)
    return result


DECODE_WORKLOAD = "moe-20b-decode-T64"


def decode_summary(args, wl):
    """The decode-shaped 20B layer (T = 64, every step reading its weights from HBM) timed the same
    way as the main workload, reduced to its HBM figures: the whole step's algorithmic bytes per
    second and the dominant kernel's (the gate_up product's weight stream)."""
    import copy
    _, cfg, flags = wl[DECODE_WORKLOAD]
    sub = copy.copy(args)
    sub.no_cpu_baseline = True
    sub.graph = False
    r = bench_moe(sub, DECODE_WORKLOAD, cfg, flags)
    st, rf = r["step"], r["roofline"]
    return {"workload": DECODE_WORKLOAD, "ms_per_step": r["ms_per_step"],
            "tokens_per_s": r["value"], "steps": r["steps"],
            "weight_copies": r["config"]["weight_copies"],
            "token_batches": r["config"]["token_batches"],
            "step_hbm_gbs_algorithmic": st["hbm_gbs_algorithmic"],
            "step_frac_of_hbm_peak": st["frac"],
            "dominant_kernel": rf["kernel"], "kernel_avg_ms": rf["avg_ms"],
            "kernel_gbs_algorithmic": rf["achieved"], "kernel_frac_of_hbm_peak": rf["frac"],
            "kernel_traffic_bytes": rf["traffic"],
            "kernels": r["kernels"]}


def settle_clocks(step, settle_ms):
    """Untimed steps until the GPU has run them for settle_ms milliseconds (by events), before the
    warm-up steps: after the setup's pauses the chip takes some milliseconds of sustained work to
    reach the clocks it then holds, and a short warm-up alone leaves the first timed steps slow
    (20B prefill: 1.640 ms per step after 5 warm-up steps, 1.578 after 20, same box).
    Returns what it did, for the output line."""
    import torch
    if settle_ms <= 0:
        return {"ms": 0.0, "steps": 0}
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    n, el, batch = 0, 0.0, 1
    a.record(stream)
    while el < settle_ms:
        for _ in range(batch):
            step(n)
            n += 1
        b.record(stream)
        b.synchronize()
        el = a.elapsed_time(b)
        batch = min(64, batch * 2)
    return {"ms": round(el, 1), "steps": n}


def host_cpu() -> str:
    """The host CPU's model name (Linux), for the baseline's description."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline_moe(args, s, x_np, wr_np, br_np, host_w, mx_act=False):
    """The oracle (router + top-k + MoE MLP) on the first tokens of the same batch, in chunks,
    until about args.cpu_seconds of wall time have passed."""
    import numpy as np
    import oracle
    chunk = max(1, min(s.T, oracle.num_threads()))
    done = 0
    t0 = time.perf_counter()
    while done < s.T and time.perf_counter() - t0 < args.cpu_seconds:
        n = min(chunk, s.T - done)
        xc = np.ascontiguousarray(x_np[done:done + n])
        lg = oracle.router_logits(xc, wr_np, br_np)
        idx, w = oracle.topk_softmax(lg, s.k)
        oracle.moe_mlp(xc, idx, w, *host_w, E=s.E, mx_act=mx_act)
        done += n
    el = time.perf_counter() - t0
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "first %d of the %d tokens: router, top-%d softmax and MoE MLP%s in the fp64 "
                      "C oracle, %.1f s wall, %d threads on %s" % (
                          done, s.T, s.k, " (activation variant)" if mx_act else "", el,
                          oracle.num_threads(), host_cpu())}


def bench_linear(args, name, cfg):
    import numpy as np
    import torch
    import mxfp4_weight_quantized_amd as mx
    from mxfp4_weight_quantized_amd import inputs
    M, K, N, seed = cfg["M"], cfg["K"], cfg["N"], cfg["seed"]
    x = _upload_bf16(inputs.activations(seed, M, K))
    w = inputs.linear_weight_f32(seed, N, K)
    p, sc = mx.mxfp4_quantize(torch.from_numpy(w).cuda())
    wbytes = N * K * 17 // 32
    n_w = max(1, math.ceil(2 * CACHE_BYTES / wbytes))
    wsets = [(p, sc)] + [(p.clone(), sc.clone()) for _ in range(n_w - 1)]
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws_bytes = mx.mxfp4_linear_workspace(M, K, N, 0)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    ws_ptr = ws.data_ptr() if ws_bytes else None
    L = mx.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step(i):
        pp, ss = wsets[i % n_w]
        st = L.mxfp4_linear(x.data_ptr(), M, K, pp.data_ptr(), ss.data_ptr(), N, out.data_ptr(),
                            mx.MX_BF16, 0, ws_ptr, ws_bytes, sh)
        if st != 0:
            raise mx.MXError(st, mx.last_error())

    settle = settle_clocks(step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    mx.mx_profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    prof = mx.mx_profile_read()
    mx.mx_profile_enable(False)
    n, tot = prof["linear"]
    avg = tot / n
    flops = 2.0 * M * K * N
    nbytes = wbytes + M * K * 2 + M * N * 2
    roof = roofline_entry(flops, nbytes, avg, PEAK_BF16_TFLOPS)
    roof.update({"traffic": read_traffic(name, "linear"), "kernel": "linear",
                 "avg_ms": round(avg, 5), "algorithmic_bytes": nbytes, "algorithmic_flops": flops})
    result = {
        "metric": METRIC, "value": round(M / (ms * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "M": M, "K": K, "N": N, "seed": seed, "weight_copies": n_w,
                   "parallelism": "single-gpu"},
        "settle": settle,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        import oracle
        xh = inputs.activations(seed, M, K)
        ph, sh_ = oracle.quantize(w)
        reps, t0c = 0, time.perf_counter()
        while time.perf_counter() - t0c < min(args.cpu_seconds, 5.0) or reps == 0:
            oracle.linear(xh, ph, sh_)
            reps += 1
        el = time.perf_counter() - t0c
        result["cpu_baseline"] = {"value": round(reps * M / el, 3), "unit": "tokens/s",
                                  "cores": oracle.num_threads(), "kind": "oracle",
                                  "sample": "%d full calls (%d tokens each), %.1f s wall, %d threads on %s"
                                            % (reps, M, el, oracle.num_threads(), host_cpu())}
    return result


def calibrate_copy(nbytes=1 << 30):
    """A plain device copy of known size, so counter runs can scale FETCH_SIZE / WRITE_SIZE."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(a, 1.0, out=b)   # reads nbytes, writes nbytes
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------------------------
def summarize_counters(fetch_dir, write_dir, copy_bytes=1 << 30):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel from two rocprofv3 --pmc
    runs of `bench.py --calibrate-copy`, scaled by what the copy kernel's counters read for its
    known traffic; writes profiles/traffic.json and prints a text summary."""
    def load(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        acc = {}
        for f in files:
            for row in csv.DictReader(open(f)):
                if row.get("Counter_Name") != counter:
                    continue
                k = row.get("Kernel_Name", "")
                acc.setdefault(k, []).append(float(row["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}
    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    copy_k = [k for k in fetch if "elementwise" in k or "copy" in k.lower()]
    if not copy_k:
        raise SystemExit("no copy kernel in the counter output")
    ck = max(copy_k, key=lambda k: fetch[k])
    f_fetch = copy_bytes / (fetch[ck] * 1024.0)
    f_write = copy_bytes / (write[ck] * 1024.0)
    # kind -> kernel symbols of one launch of it (the router is two kernels: the 64-token tile
    # kernel or the spread logits kernel, then the selection; the set-up's routing of every batch,
    # outside the timed region, runs the logits kernel's selecting form, which is left out)
    router = (["route_tile_kernel"] if any("route_tile_kernel" in k for k in fetch)
              else ["route_logits_kernel<false"])
    kinds = {"moe_gate_up_swiglu": ["moe_gate_up_swiglu_kernel"],
             "moe_down_weighted": ["moe_down_weighted_kernel"], "moe_combine": ["combine_token_kernel"],
             "route_topk": router + ["route_select_kernel"],
             "permute": ["permute_kernel", "slice_hist_kernel", "slice_scatter_kernel"],
             "linear": ["linear_kernel"],
             "quantize": ["quantize_kernel<true>", "x_pair_copy_kernel", "quantize_x_scatter_kernel"],
             "moe_single_launch": ["moe_single_launch_kernel"]}
    out = {}
    for kind, syms in kinds.items():
        fk = wk = 0.0
        found = False
        for sym in syms:
            ks = [k for k in fetch if sym in k]
            if not ks:
                continue
            found = True
            fk += sum(fetch[k] for k in ks) / len(ks)
            wk += sum(write.get(k, 0.0) for k in ks) / len(ks)
        if not found:
            continue
        out[kind] = {"fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                     "hbm_bytes_per_launch": int(fk * 1024 * f_fetch + wk * 1024 * f_write),
                     "copy_scale_fetch": round(f_fetch, 4), "copy_scale_write": round(f_write, 4),
                     "source_sha": source_sha()}
    return out


def summarize_traffic(workload, bench_json, commands):
    """Markdown table of the counted HBM bytes per launch of one workload (from traffic.json)
    beside the algorithmic bytes the bench line of the same workload reports per kernel."""
    ent = json.load(open(TRAFFIC_FILE))[workload]
    kern = json.load(open(bench_json)).get("kernels", {})
    any_k = next(iter(ent.values()))
    out = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE): %s" % workload, "",
           "Commands (the profiler runs from /tmp with TMPDIR=/tmp and writes under the -d "
           "directory; REPO is the repository root):", "", "```"] + list(commands) + [
           "```", "",
           "`--calibrate-copy` appends a 1 GiB elementwise copy (reads 1 GiB, writes 1 GiB); its "
           "counters give the scale factors: fetch KiB x %.4f, write KiB x %.4f. Averages over "
           "every launch of the kernel in the run. Algorithmic bytes: what the kernel must read "
           "and write once (the bench line's per-kernel `bytes`)."
           % (any_k["copy_scale_fetch"], any_k["copy_scale_write"]), "",
           "| kernel | fetch KiB | write KiB | HBM MB / launch | algorithmic MB | ratio |",
           "|---|---:|---:|---:|---:|---:|"]
    for k, v in sorted(ent.items(), key=lambda kv: -kv[1]["hbm_bytes_per_launch"]):
        if kern and k not in kern:  # (a kernel of the set-up, such as the weights' quantization)
            continue
        alg = kern.get(k, {}).get("bytes")
        out.append("| %s | %s | %s | %.1f | %s | %s |" % (
            k, format(v["fetch_kib"], ",.0f"), format(v["write_kib"], ",.0f"),
            v["hbm_bytes_per_launch"] / 1e6, "%.1f" % (alg / 1e6) if alg else "-",
            "%.2f" % (v["hbm_bytes_per_launch"] / alg) if alg else "-"))
    out += ["", "Library sources: `%s` (hash of csrc/; the bench reports `traffic` only while "
            "it matches)." % any_k["source_sha"]]
    return "\n".join(out) + "\n"


def summarize_mfma(pmc_dir, command, title):
    """Markdown table of MFMA activity per dispatch of the grouped GEMMs from a rocprofv3 --pmc run
    of GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES and SQ_INSTS_MFMA (with dispatch timestamps).
    GRBM_GUI_ACTIVE is summed over the 8 XCDs and SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs:
    cycles per XCD over the dispatch time is the clock the chip held, and busy cycles per SIMD
    over that the share of cycles the matrix pipes were busy."""
    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % pmc_dir)
    disp = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            d = disp.setdefault((f, r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                        "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = ["# %s" % title, "", "Command (run from /tmp with TMPDIR=/tmp, output under the -d "
           "directory; REPO is the repository root):", "", "```", command, "```", "",
           "Per-dispatch averages. GRBM_GUI_ACTIVE is summed over the 8 XCDs (cycles per XCD over "
           "the dispatch time = the clock the chip held); SQ_VALU_MFMA_BUSY_CYCLES over the 1 024 "
           "SIMDs (busy cycles per SIMD over the cycles = the share of cycles the matrix pipes were "
           "busy).", "",
           "| kernel | dispatches | avg us | clock MHz | MFMA instructions | MFMA busy | busy x clock / 2.4 GHz |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for sym in ("moe_gate_up_swiglu_kernel", "moe_down_weighted_kernel"):
        ds = [d for d in disp.values() if sym in d["name"] and "GRBM_GUI_ACTIVE" in d]
        if not ds:
            continue
        ns = sum(d["ns"] for d in ds) / len(ds)
        cyc = sum(d["GRBM_GUI_ACTIVE"] for d in ds) / len(ds) / 8.0
        busy = sum(d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for d in ds) / len(ds) / 1024.0
        ins = sum(d.get("SQ_INSTS_MFMA", 0.0) for d in ds) / len(ds)
        mhz = cyc / ns * 1e3
        frac = busy / cyc if cyc else 0.0
        out.append("| `%s` | %d | %.1f | %.0f | %.2fM | %.1f %% | %.1f %% |" % (
            sym, len(ds), ns / 1e3, mhz, ins / 1e6, 100 * frac, 100 * frac * mhz / 2400.0))
    out.append("")
    out.append("Library sources: `%s` (hash of csrc/)." % source_sha())
    return "\n".join(out) + "\n"


def summarize_vmem(command, title, dirs):
    """Markdown table of the vector memory pipeline per dispatch of the MoE kernels from rocprofv3
    --pmc runs (one directory per workload, named pmc_ta_<workload>) of GRBM_GUI_ACTIVE, the TA and
    TD busy and L1-stall counters, the L1's pending and tag-conflict stalls and its L2 read
    requests with their summed latency. GRBM_GUI_ACTIVE is summed over the 8 XCDs, the TA, TD and
    TCP counters over the 256 CUs: each of those is shown as a share of 256 x the dispatch's
    cycles per XCD."""
    out = ["# %s" % title, "", "Command per workload (run from /tmp with TMPDIR=/tmp, output under "
           "the -d directory; REPO is the repository root; WL = %s):" % ", then ".join(
               os.path.basename(d.rstrip("/")).replace("pmc_ta_", "") for d in dirs), "", "```",
           command, "```", "",
           "Per-dispatch averages. L2 latency = TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ (cycles "
           "per L1 -> L2 read request). Library sources: `%s` (hash of csrc/)." % source_sha(), "",
           "| workload | kernel | dispatches | avg us | TA busy | TA stalled by L1 | TD busy | "
           "TD stalled by L1 | L1 pending stall | L1 tag conflict | L2 latency (cycles) | "
           "L1->L2 requests |",
           "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for d in dirs:
        wl = os.path.basename(d.rstrip("/")).replace("pmc_ta_", "")
        disp = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                e = disp.setdefault((f, r["Dispatch_Id"]), {
                    "name": r["Kernel_Name"], "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for sym in ("moe_gate_up_swiglu_kernel", "moe_down_weighted_kernel", "combine_token_kernel"):
            ds = [e for e in disp.values() if sym in e["name"] and "GRBM_GUI_ACTIVE" in e]
            if not ds:
                continue
            avg = lambda c: sum(e.get(c, 0.0) for e in ds) / len(ds)
            cu = 256.0 * avg("GRBM_GUI_ACTIVE") / 8.0
            pct = lambda c: "%.1f %%" % (100.0 * avg(c) / cu)
            req = avg("TCP_TCC_READ_REQ")
            out.append("| %s | `%s` | %d | %.1f | %s | %s | %s | %s | %s | %s | %.0f | %.1fM |" % (
                wl, sym, len(ds), avg("ns") / 1e3, pct("TA_TA_BUSY"),
                pct("TA_ADDR_STALLED_BY_TC_CYCLES"), pct("TD_TD_BUSY"), pct("TD_TC_STALL"),
                pct("TCP_PENDING_STALL_CYCLES"), pct("TCP_READ_TAGCONFLICT_STALL_CYCLES"),
                avg("TCP_TCC_READ_REQ_LATENCY") / req if req else float("nan"), req / 1e6))
    return "\n".join(out) + "\n"


def summarize_trace(trace_dir, command, title, bench_json=None):
    """Markdown table of a rocprofv3 --kernel-trace --stats run (its *kernel_stats.csv): calls,
    average / min / max duration and share of GPU time per kernel; with bench_json (the traced
    bench.py run's own output line), the step time and the dominant kernel by HIP events next
    to the trace's figure for it."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_stats.csv under %s" % trace_dir)
    rows = list(csv.DictReader(open(files[0])))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["# %s" % title, "", "Command (run from /tmp with TMPDIR=/tmp, output under the -d "
           "directory; REPO is the repository root):", "", "```", command, "```", "",
           "| kernel | calls | avg us | min us | max us | share % |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"].replace("mx::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        out.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f |" % (
            name[:110], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    if bench_json:
        b = json.loads(open(bench_json).read().strip().splitlines()[-1])
        roof = b.get("roofline", {})
        dom = roof.get("kernel")
        sym = {"moe_gate_up_swiglu": "moe_gate_up_swiglu_kernel", "moe_down_weighted":
               "moe_down_weighted_kernel", "moe_combine": "combine_token_kernel", "linear": "linear_kernel",
               "moe_single_launch": "moe_single_launch_kernel"}
        tr = [r for r in rows if sym.get(dom, "?") in r["Name"]]
        out += ["", "The traced bench.py run's own line: %.4f ms per step; dominant kernel `%s` "
                "%.2f us by HIP events (%s), %.2f us in this trace (all calls, warm-up included)."
                % (b["ms_per_step"], dom, roof.get("avg_ms", 0) * 1e3,
                   "%.1f %s = %.1f %% of peak" % (roof.get("achieved", 0), roof.get("unit", ""),
                                                  100 * roof.get("frac", 0)),
                   float(tr[0]["AverageNs"]) / 1e3 if tr else float("nan")),
                "Library sources: `%s` (hash of csrc/, as in the bench's traffic lookup)."
                % source_sha()]
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first: the clocks settle over the first ~10 ms of work")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed steps for this long before the warm-up steps (clock settling)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="default workload only: leave out the decode layer's line")
    ap.add_argument("--graph", action="store_true",
                    help="replay the steps from a HIP graph instead of launching them one by one")
    ap.add_argument("--row-major-weights", action="store_true",
                    help="feed the grouped GEMMs row-major weights instead of the tiled layout")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (for counter scaling)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--traffic-workload", default=None,
                    help="with --summarize-counters: workload name to file the numbers under")
    ap.add_argument("--summarize-trace", nargs="+", metavar="ARG",
                    help="TRACE_DIR COMMAND TITLE [BENCH_JSON]: print a markdown summary of a "
                         "rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--summarize-traffic", nargs="+",
                    metavar="WORKLOAD BENCH_JSON [COMMAND ...]",
                    help="print a markdown table of the committed counter traffic of a workload")
    ap.add_argument("--summarize-vmem", nargs="+", metavar="ARG",
                    help="COMMAND TITLE DIR [DIR ...]: markdown summary of vector memory counters")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("PMC_DIR", "COMMAND", "TITLE"),
                    help="print a markdown summary of the MFMA counters of a rocprofv3 --pmc run")
    args = ap.parse_args()

    if args.summarize_trace:
        sys.stdout.write(summarize_trace(*args.summarize_trace))
        return 0

    if args.summarize_traffic:
        wl_, bj = args.summarize_traffic[:2]
        sys.stdout.write(summarize_traffic(wl_, bj, args.summarize_traffic[2:]))
        return 0

    if args.summarize_vmem:
        sys.stdout.write(summarize_vmem(args.summarize_vmem[0], args.summarize_vmem[1],
                                        args.summarize_vmem[2:]))
        return 0

    if args.summarize_mfma:
        sys.stdout.write(summarize_mfma(*args.summarize_mfma))
        return 0

    if args.summarize_counters:
        wl = args.traffic_workload or args.workload
        res = summarize_counters(*args.summarize_counters)
        data = {}
        if os.path.exists(TRAFFIC_FILE):
            data = json.load(open(TRAFFIC_FILE))
        data[wl] = res
        os.makedirs(PROFILES, exist_ok=True)
        json.dump(data, open(TRAFFIC_FILE, "w"), indent=1, sort_keys=True)
        print(json.dumps({wl: res}, indent=1))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        return 2
    wl = workloads()
    if args.workload not in wl:
        print("unknown workload %s; choose from %s" % (args.workload, sorted(wl)), file=sys.stderr)
        return 2
    kind, cfg, flags = wl[args.workload]
    if kind == "moe":
        res = bench_moe(args, args.workload, cfg, flags)
        if args.workload == DEFAULT_WORKLOAD and not args.no_decode:
            res["decode"] = decode_summary(args, wl)
    else:
        res = bench_linear(args, args.workload, cfg)
    if args.calibrate_copy:
        calibrate_copy()
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
