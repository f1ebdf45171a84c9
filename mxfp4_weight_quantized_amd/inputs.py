"""Seeded synthetic inputs for the MXFP4 MoE-MLP path, shared by the tests and the benchmark.

This module holds no arithmetic of the method: it only draws random numbers and casts them to the
storage dtypes (bf16 by torch's round-to-nearest-even cast). Quantization of the drawn fp32
weights is left to the caller (the oracle in tests, the HIP library in the benchmark).

Recipe: every tensor has its own numpy PCG64 stream keyed by (seed, tag, sub-index), so a tensor's
values do not depend on what else was drawn or in which order. Draws are fp32 standard normals
times the standard deviation.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

TAG_X = 1          # activations, sub-index = T
TAG_ROUTER_W = 2   # router weight
TAG_ROUTER_B = 3   # router bias
TAG_GATE_UP = 4    # expert gate_up weight, sub-index = expert
TAG_DOWN = 5       # expert down weight, sub-index = expert
TAG_LINEAR_W = 6   # dense linear weight
TAG_MISC = 7       # anything else a test draws (sub-index chosen by the test)

WEIGHT_STD = 0.02


def rng(seed: int, tag: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tag), int(sub)])


def normal_f32(seed: int, tag: int, shape, std: float = 1.0, sub: int = 0) -> np.ndarray:
    a = rng(seed, tag, sub).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(seed: int, T: int, H: int, std: float = 1.0) -> np.ndarray:
    """bf16 bits [T, H], ~N(0, std)."""
    return bf16_bits(normal_f32(seed, TAG_X, (T, H), std, sub=T))


def router(seed: int, E: int, H: int, bias_std: float = 0.0):
    """(W_r bf16 bits [E, H] ~N(0, 0.02), b_r fp32 [E] ~N(0, bias_std) or zeros)."""
    wr = bf16_bits(normal_f32(seed, TAG_ROUTER_W, (E, H), WEIGHT_STD))
    if bias_std > 0:
        br = normal_f32(seed, TAG_ROUTER_B, (E,), bias_std)
    else:
        br = np.zeros(E, np.float32)
    return wr, br


def gate_up_f32(seed: int, e: int, F: int, H: int) -> np.ndarray:
    """Expert e's gate_up weight, fp32 [2F, H] (rows [0, F) gate, [F, 2F) up)."""
    return normal_f32(seed, TAG_GATE_UP, (2 * F, H), WEIGHT_STD, sub=e)


def down_f32(seed: int, e: int, H: int, F: int) -> np.ndarray:
    """Expert e's down weight, fp32 [H, F]."""
    return normal_f32(seed, TAG_DOWN, (H, F), WEIGHT_STD, sub=e)


def linear_weight_f32(seed: int, N: int, K: int) -> np.ndarray:
    return normal_f32(seed, TAG_LINEAR_W, (N, K), WEIGHT_STD)


def expert_weights(seed: int, E: int, H: int, F: int, quantize, threads: int = 8):
    """Draw all experts' weights and pack them with ``quantize`` (fp32 [R, K] -> (packed, scales)).

    Returns (gu_packed [E, 2F, H/2], gu_scales [E, 2F, H/32], dn_packed [E, H, F/2],
    dn_scales [E, H, F/32]) as numpy uint8 arrays. The random draws run on ``threads`` worker
    threads, at most ``threads`` experts ahead, so the fp32 copies never all coexist;
    ``quantize`` is called on the calling thread only (it may run its own thread team)."""
    gu_p = np.empty((E, 2 * F, H // 2), np.uint8)
    gu_s = np.empty((E, 2 * F, H // 32), np.uint8)
    dn_p = np.empty((E, H, F // 2), np.uint8)
    dn_s = np.empty((E, H, F // 32), np.uint8)

    def draw(e):
        return gate_up_f32(seed, e, F, H), down_f32(seed, e, H, F)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        pending = [ex.submit(draw, e) for e in range(min(E, max(1, threads)))]
        for e in range(E):
            wgu, wdn = pending[e].result()
            pending[e] = None
            if len(pending) < E:  # keep `threads` draws in flight
                pending.append(ex.submit(draw, len(pending)))
            gu_p[e], gu_s[e] = quantize(wgu)
            dn_p[e], dn_s[e] = quantize(wdn)
    return gu_p, gu_s, dn_p, dn_s


@dataclass(frozen=True)
class MoEShape:
    name: str
    T: int
    H: int
    F: int
    E: int
    k: int
    seed: int
    bias_std: float = 0.0


# The workloads the path is sized for (gpt-oss-style MoE layers, hidden 2880, expert FFN 2880,
# top-4) plus the small shapes the oracle finishes in seconds.
MOE_20B_DECODE = MoEShape("moe-20b-decode-T64", T=64, H=2880, F=2880, E=32, k=4, seed=2)
MOE_20B_PREFILL = MoEShape("moe-20b-prefill-T8192-skewed", T=8192, H=2880, F=2880, E=32, k=4,
                           seed=3, bias_std=0.5)
MOE_120B = {T: MoEShape("moe-120b-T%d" % T, T=T, H=2880, F=2880, E=128, k=4, seed=4)
            for T in (1, 256, 4096)}
