"""CPU oracle for the MXFP4 weight-quantized MoE MLP (plain C, fp64), with numpy wrappers.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never imports, links or calls it, and it
shares no code with the HIP library.

The arithmetic lives in ``mx_oracle.c``; this module only builds it with gcc, loads it with
ctypes and marshals numpy arrays. Each wrapper names the C function it calls; the C source cites
the page passage each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mx_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmx_oracle.so")
# A test that plants mistakes in copies of the oracle points this at a mutant build.
_LIB_OVERRIDE = os.environ.get("MXO_ORACLE_LIB")
_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-pthread", "-fPIC",
             "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile ``mx_oracle.c`` (or another source, e.g. a planted-mistake copy) with gcc."""
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *GCC_FLAGS, "-I", _HERE, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(tmp, out)
    return out


def _P(t):
    return ctypes.POINTER(t)


class ActParams(ctypes.Structure):
    """Mirror of mxo_act_params (the expert activation's parameters)."""
    _fields_ = [("interleaved", ctypes.c_int), ("alpha", ctypes.c_double),
                ("limit", ctypes.c_double), ("up_shift", ctypes.c_double),
                ("gu_bias", ctypes.POINTER(ctypes.c_float)),
                ("dn_bias", ctypes.POINTER(ctypes.c_float))]


def lib():
    """Load the oracle library, building it first if it is not there."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
                    os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "mx_oracle.h"))):
                build()
            L = ctypes.CDLL(_LIB_PATH)
        u8, u16, i32, f32, f64 = (ctypes.c_uint8, ctypes.c_uint16, ctypes.c_int32,
                                  ctypes.c_float, ctypes.c_double)
        i64, c_int = ctypes.c_int64, ctypes.c_int
        sig = {
            "mxo_e2m1_value": (f64, [ctypes.c_uint]),
            "mxo_e8m0_value": (f64, [ctypes.c_uint]),
            "mxo_weight_operand": (f64, [ctypes.c_uint, ctypes.c_uint, c_int]),
            "mxo_bf16_from_double": (u16, [f64]),
            "mxo_double_from_bf16": (f64, [u16]),
            "mxo_quantize_f32": (None, [_P(f32), i64, i64, _P(u8), _P(u8)]),
            "mxo_quantize_bf16": (None, [_P(u16), i64, i64, _P(u8), _P(u8)]),
            "mxo_dequantize": (None, [_P(u8), _P(u8), i64, i64, _P(f64)]),
            "mxo_router_logits": (None, [_P(u16), _P(u16), _P(f32), c_int, c_int, c_int, _P(f32)]),
            "mxo_topk_softmax": (None, [_P(f32), c_int, c_int, c_int, _P(i32), _P(f32)]),
            "mxo_permute": (c_int, [_P(i32), c_int, c_int, c_int, _P(i32), _P(i32), _P(i32)]),
            "mxo_linear": (None, [_P(u16), c_int, c_int, _P(u8), _P(u8), c_int, c_int, _P(f64)]),
            "mxo_moe_mlp": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, _P(u16), _P(i32),
                                    _P(f32), _P(u8), _P(u8), _P(u8), _P(u8), _P(i32), c_int,
                                    _P(f64), _P(u16)]),
            "mxo_moe_mlp_ex": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, _P(u16), _P(i32),
                                       _P(f32), _P(u8), _P(u8), _P(u8), _P(u8), _P(i32), c_int,
                                       _P(f64), _P(u16), f64, _P(u16), _P(f64)]),
            "mxo_moe_mlp_act": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, _P(u16), _P(i32),
                                        _P(f32), _P(u8), _P(u8), _P(u8), _P(u8), _P(i32), c_int,
                                        _P(f64), _P(u16), f64, _P(u16), _P(f64),
                                        ctypes.POINTER(ActParams)]),
            "mxo_num_threads": (c_int, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
        return L


def _ptr(a: np.ndarray | None, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _as(a, dtype):
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


# ----------------------------------------------------------------------------------------------
# numpy-level wrappers (bf16 tensors travel as uint16 bit patterns)
# ----------------------------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    """mxo_e2m1_value: value of a 4-bit E2M1 code."""
    return lib().mxo_e2m1_value(int(code))


def e8m0_value(b: int) -> float:
    """mxo_e8m0_value: 2^(b-127), NaN for 255."""
    return lib().mxo_e8m0_value(int(b))


def weight_operand(code: int, b: int, mx_act: bool = False) -> float:
    """mxo_weight_operand: value of weight element (code, scale byte b) in the matrix products
    (the bf16 operand for bf16 activations, the exact value for the activation variant)."""
    return lib().mxo_weight_operand(int(code), int(b), int(bool(mx_act)))


def bf16_from_double(d: float) -> int:
    """mxo_bf16_from_double: single round-to-nearest-even step from fp64 to bf16 bits."""
    return int(lib().mxo_bf16_from_double(float(d)))


def quantize(src: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """mxo_quantize_f32 / mxo_quantize_bf16: rows of K along K in 32-blocks.

    ``src`` is float32 [R, K] or uint16 (bf16 bits) [R, K]. Returns (packed uint8 [R, K/2],
    scales uint8 [R, K/32])."""
    src = np.asarray(src)
    R, K = src.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    packed = np.zeros((R, K // 2), np.uint8)
    scales = np.zeros((R, K // 32), np.uint8)
    if src.dtype == np.uint16:
        s = _as(src, np.uint16)
        lib().mxo_quantize_bf16(_ptr(s, ctypes.c_uint16), R, K, _ptr(packed, ctypes.c_uint8),
                                _ptr(scales, ctypes.c_uint8))
    else:
        s = _as(src, np.float32)
        lib().mxo_quantize_f32(_ptr(s, ctypes.c_float), R, K, _ptr(packed, ctypes.c_uint8),
                               _ptr(scales, ctypes.c_uint8))
    return packed, scales


def dequantize(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """mxo_dequantize: exact fp64 values of a packed [R, K/2] + scales [R, K/32] tensor."""
    packed = _as(packed, np.uint8)
    scales = _as(scales, np.uint8)
    R = packed.shape[0]
    K = packed.shape[1] * 2
    out = np.zeros((R, K), np.float64)
    lib().mxo_dequantize(_ptr(packed, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8), R, K,
                         _ptr(out, ctypes.c_double))
    return out


def router_logits(x_bf16, wr_bf16, br=None) -> np.ndarray:
    """mxo_router_logits: fp32 logits [T, E]."""
    x = _as(x_bf16, np.uint16)
    wr = _as(wr_bf16, np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    b = None if br is None else _as(br, np.float32)
    out = np.zeros((T, E), np.float32)
    lib().mxo_router_logits(_ptr(x, ctypes.c_uint16), _ptr(wr, ctypes.c_uint16),
                            _ptr(b, ctypes.c_float), T, H, E, _ptr(out, ctypes.c_float))
    return out


def topk_softmax(logits, k: int) -> tuple[np.ndarray, np.ndarray]:
    """mxo_topk_softmax: (idx int32 [T, k], w float32 [T, k])."""
    l = _as(logits, np.float32)
    T, E = l.shape
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float32)
    lib().mxo_topk_softmax(_ptr(l, ctypes.c_float), T, E, k, _ptr(idx, ctypes.c_int32),
                           _ptr(w, ctypes.c_float))
    return idx, w


def permute(idx, E: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """mxo_permute: (offsets int32 [E+1], perm int32 [T*k], inv int32 [T*k])."""
    i = _as(idx, np.int32)
    T, k = i.shape
    offsets = np.zeros(E + 1, np.int32)
    perm = np.zeros(T * k, np.int32)
    inv = np.zeros(T * k, np.int32)
    rc = lib().mxo_permute(_ptr(i, ctypes.c_int32), T, k, E, _ptr(offsets, ctypes.c_int32),
                           _ptr(perm, ctypes.c_int32), _ptr(inv, ctypes.c_int32))
    if rc != 0:
        raise ValueError("expert index out of range")
    return offsets, perm, inv


def linear(x_bf16, packed, scales, mx_act: bool = False) -> np.ndarray:
    """mxo_linear: fp64 Y [M, N] = X W^T."""
    x = _as(x_bf16, np.uint16)
    M, K = x.shape
    p = _as(packed, np.uint8)
    s = _as(scales, np.uint8)
    N = p.shape[0]
    y = np.zeros((M, N), np.float64)
    lib().mxo_linear(_ptr(x, ctypes.c_uint16), M, K, _ptr(p, ctypes.c_uint8),
                     _ptr(s, ctypes.c_uint8), N, int(bool(mx_act)), _ptr(y, ctypes.c_double))
    return y


def moe_mlp(x_bf16, topk_idx, topk_w, gu_packed, gu_scales, dn_packed, dn_scales, E: int,
            tokens=None, mx_act: bool = False, want_h: bool = False, fragile_c: float | None = None,
            act: dict | None = None):
    """mxo_moe_mlp: fp64 output rows [n_tokens, H] (and optionally the bf16 h rows).

    Shapes: x [T, H] bf16 bits; topk_idx/topk_w [T, k]; gu_packed [E, 2F, H/2]; gu_scales
    [E, 2F, H/32]; dn_packed [E, H, F/2]; dn_scales [E, H, F/32].

    fragile_c (activation variant): also return (h_alt [n, k, F], slack [n, H]) from
    mxo_moe_mlp_ex -- the h quantization decisions an fp32 implementation may take the other
    way, with fp32 errors of g and u assumed below fragile_c * 2^-24 * sqrt(H * sum terms^2),
    and the bound on the output change they can cause. Returned as (out, [h,] h_alt, slack).

    act (mxo_moe_mlp_act): the expert activation's parameters, a dict with any of interleaved
    (bool), alpha, limit, up_shift (floats) and gu_bias [E, 2F], dn_bias [E, H] (fp32 arrays);
    None = the plain SwiGLU."""
    x = _as(x_bf16, np.uint16)
    T, H = x.shape
    idx = _as(topk_idx, np.int32)
    w = _as(topk_w, np.float32)
    k = idx.shape[1]
    gp, gs = _as(gu_packed, np.uint8), _as(gu_scales, np.uint8)
    dp, ds = _as(dn_packed, np.uint8), _as(dn_scales, np.uint8)
    F = dp.shape[-1] * 2
    assert gp.size == E * 2 * F * H // 2 and dp.size == E * H * F // 2
    tok = None if tokens is None else _as(tokens, np.int32)
    n = T if tok is None else tok.shape[0]
    out = np.zeros((n, H), np.float64)
    h = np.zeros((n, k, F), np.uint16) if want_h else None
    args = (T, H, F, E, k, int(bool(mx_act)), _ptr(x, ctypes.c_uint16), _ptr(idx, ctypes.c_int32),
            _ptr(w, ctypes.c_float), _ptr(gp, ctypes.c_uint8), _ptr(gs, ctypes.c_uint8),
            _ptr(dp, ctypes.c_uint8), _ptr(ds, ctypes.c_uint8), _ptr(tok, ctypes.c_int32), n,
            _ptr(out, ctypes.c_double), _ptr(h, ctypes.c_uint16))
    h_alt = slack = None
    if fragile_c is not None:
        h_alt = np.zeros((n, k, F), np.uint16)
        slack = np.zeros((n, H), np.float64)
    if act is None:
        if fragile_c is None:
            rc = lib().mxo_moe_mlp(*args)
        else:
            rc = lib().mxo_moe_mlp_ex(*args, float(fragile_c), _ptr(h_alt, ctypes.c_uint16),
                                      _ptr(slack, ctypes.c_double))
    else:
        gb = None if act.get("gu_bias") is None else _as(act["gu_bias"], np.float32)
        db = None if act.get("dn_bias") is None else _as(act["dn_bias"], np.float32)
        assert gb is None or gb.size == E * 2 * F
        assert db is None or db.size == E * H
        ap = ActParams(int(bool(act.get("interleaved", False))), float(act.get("alpha", 0.0)),
                       float(act.get("limit", 0.0)), float(act.get("up_shift", 0.0)),
                       _ptr(gb, ctypes.c_float), _ptr(db, ctypes.c_float))
        rc = lib().mxo_moe_mlp_act(*args, float(fragile_c or 0.0), _ptr(h_alt, ctypes.c_uint16),
                                   _ptr(slack, ctypes.c_double), ctypes.byref(ap))
    if rc != 0:
        raise ValueError("expert index out of range")
    res = [out] + ([h] if want_h else [])
    if fragile_c is not None:
        res += [h_alt, slack]
    return tuple(res) if len(res) > 1 else out


def num_threads() -> int:
    """mxo_num_threads: OpenMP threads the oracle runs with."""
    return int(lib().mxo_num_threads())
