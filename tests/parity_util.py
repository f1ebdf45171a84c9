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


def check_bf16_output(got_bits: np.ndarray, ref: np.ndarray, what: str = "", slack=None):
    """bf16 output: within one bf16 ulp of the oracle value per element, and the Frobenius bound
    (after the fragile-decision slack, if given, as in check_tolerance)."""
    got = inputs.bf16_to_f32(got_bits).astype(np.float64)
    ref = np.asarray(ref, np.float64)
    err = got - ref
    if slack is not None:
        err = np.sign(err) * np.maximum(np.abs(err) - np.asarray(slack, np.float64), 0.0)
    ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(ref), 1e-38))).astype(np.int64) - 7)
    rms = np.linalg.norm(ref, axis=-1, keepdims=True) / np.sqrt(ref.shape[-1])
    bound = np.maximum(ulp, PER_ELEM * (rms + PER_ELEM_FLOOR) * 0.1)
    bad = np.abs(err) > bound
    assert not bad.any(), "%s: %d bf16 elements off by more than one ulp" % (what, int(bad.sum()))
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= REL_FROB, "%s: relative Frobenius error %.3e" % (what, rel)


@functools.lru_cache(maxsize=4)
def moe_weights(seed: int, E: int, H: int, F: int):
    """Oracle-packed expert weights for a (seed, E, H, F) layer, on the host."""
    return inputs.expert_weights(seed, E, H, F, oracle.quantize, threads=4)


@functools.lru_cache(maxsize=4)
def moe_weights_dev(seed: int, E: int, H: int, F: int):
    return tuple(to_dev(a) for a in moe_weights(seed, E, H, F))
