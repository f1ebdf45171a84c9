"""MXFP4 weight-quantized MoE MLP for MI355X (gfx950): thin Python binding of the C ABI.

The functions here carry the names of the C entry points in ``include/mxfp4moe.h`` and only
marshal arguments: torch supplies device memory and the current stream, and every step of the
computation runs in the HIP library ``libmxfp4moe.so``. There is no CPU fallback: if the library
is missing or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxfp4moe.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "mxfp4moe.h")

MX_OK, MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_DTYPE = 0, 1, 2, 3, 4
MX_ERR_WORKSPACE, MX_ERR_UNSUPPORTED, MX_ERR_HIP = 5, 6, 7
MX_F32, MX_BF16 = 0, 1
MX_ACT_MXFP4 = 0x1
MX_WEIGHTS_TILED = 0x2
MX_SINGLE_LAUNCH = 0x4
MX_DEVERR_ROUTING = 0x1
MX_DEVERR_SYNC = 0x2
MX_NOALLOC_SCRATCH_BYTES = 32 << 20
MX_GU_INTERLEAVED = 0x1
MX_TILE_DEINTERLEAVE = 0x1
STATUS_NAMES = {0: "MX_OK", 1: "MX_ERR_NULL", 2: "MX_ERR_SHAPE", 3: "MX_ERR_ALIGN",
                4: "MX_ERR_DTYPE", 5: "MX_ERR_WORKSPACE", 6: "MX_ERR_UNSUPPORTED", 7: "MX_ERR_HIP"}


class MXError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))
        self.status = status


class KernelTime(ctypes.Structure):
    """Mirror of ``mx_kernel_time``."""
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double)]


class MoeDesc(ctypes.Structure):
    """Mirror of ``mx_moe_desc``."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("F", ctypes.c_int32),
        ("E", ctypes.c_int32), ("k", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("out_dtype", ctypes.c_int),
        ("x", ctypes.c_void_p), ("wr", ctypes.c_void_p), ("br", ctypes.c_void_p),
        ("topk_idx_in", ctypes.c_void_p), ("topk_w_in", ctypes.c_void_p),
        ("gu_packed", ctypes.c_void_p), ("gu_scales", ctypes.c_void_p),
        ("dn_packed", ctypes.c_void_p), ("dn_scales", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("topk_idx_out", ctypes.c_void_p), ("topk_w_out", ctypes.c_void_p),
        ("logits_out", ctypes.c_void_p),
        ("act_flags", ctypes.c_uint32), ("swiglu_alpha", ctypes.c_float),
        ("swiglu_limit", ctypes.c_float), ("swiglu_up_shift", ctypes.c_float),
        ("gu_bias", ctypes.c_void_p), ("dn_bias", ctypes.c_void_p),
    ]


_lock = threading.Lock()
_lib = None

_VP, _I32, _I64, _U32, _SZ, _INT = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                    ctypes.c_uint32, ctypes.c_size_t, ctypes.c_int)
SIGNATURES = {
    "mxfp4_quantize": (_INT, [_VP, _INT, _I64, _I64, _VP, _VP, _VP]),
    "mxfp4_dequantize": (_INT, [_VP, _VP, _I64, _I64, _VP, _INT, _VP]),
    "mxfp4_tile_weights": (_INT, [_VP, _VP, _I64, _I64, _I64, _VP, _VP, _VP]),
    "mxfp4_tile_weights_ex": (_INT, [_VP, _VP, _I64, _I64, _I64, _U32, _VP, _VP, _VP]),
    "moe_route_topk": (_INT, [_VP, _VP, _VP, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP]),
    "moe_permute_workspace": (_SZ, [_I32, _I32, _I32]),
    "moe_permute": (_INT, [_VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "mxfp4_moe_mlp_workspace": (_SZ, [ctypes.POINTER(MoeDesc)]),
    "mxfp4_moe_mlp": (_INT, [ctypes.POINTER(MoeDesc), _VP, _SZ, _VP]),
    "mxfp4_moe_mlp_noalloc": (_INT, [ctypes.POINTER(MoeDesc), _VP]),
    "mxfp4_linear_workspace": (_SZ, [_I32, _I32, _I32, _U32]),
    "mxfp4_linear": (_INT, [_VP, _I32, _I32, _VP, _VP, _I32, _VP, _INT, _U32, _VP, _SZ, _VP]),
    "mx_last_error": (ctypes.c_char_p, []),
    "mx_get_device_error": (_INT, [_VP, ctypes.POINTER(ctypes.c_int32)]),
    "mx_workspace_status": (_INT, [_VP, _VP, ctypes.POINTER(ctypes.c_int32)]),
    "mx_version": (ctypes.c_char_p, []),
    "mx_profile_enable": (_INT, [_INT]),
    "mx_profile_read": (_I32, [ctypes.POINTER(KernelTime), _I32]),
}


def lib():
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("HIP library %s is not built; run "
                                   "`python -m mxfp4_weight_quantized_amd.build`" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)  # torch is imported first, so its HIP runtime is the one used
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
        return _lib


def last_error() -> str:
    return lib().mx_last_error().decode()


def _check(status: int):
    if status != MX_OK:
        raise MXError(status, last_error())


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU (no CPU path)")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _dt(dtype) -> int:
    if dtype == torch.float32:
        return MX_F32
    if dtype == torch.bfloat16:
        return MX_BF16
    raise ValueError("dtype must be torch.float32 or torch.bfloat16")


# ---------------------------------------------------------------------------------------------
def mxfp4_quantize(src: torch.Tensor, packed=None, scales=None, stream=None):
    """src [R, K] fp32/bf16 -> (packed uint8 [R, K/2], scales uint8 [R, K/32])."""
    R, K = src.shape
    if packed is None:
        packed = torch.empty((R, K // 2), dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty((R, K // 32), dtype=torch.uint8, device=src.device)
    _check(lib().mxfp4_quantize(_ptr(src), _dt(src.dtype), R, K, _ptr(packed), _ptr(scales),
                                _stream(stream)))
    return packed, scales


def mxfp4_dequantize(packed: torch.Tensor, scales: torch.Tensor, dtype=torch.float32, out=None,
                     stream=None):
    """packed [R, K/2], scales [R, K/32] -> [R, K] in ``dtype``."""
    R = packed.shape[0]
    K = packed.shape[-1] * 2
    if out is None:
        out = torch.empty((R, K), dtype=dtype, device=packed.device)
    _check(lib().mxfp4_dequantize(_ptr(packed), _ptr(scales), R, K, _ptr(out), _dt(out.dtype),
                                  _stream(stream)))
    return out


def mxfp4_tile_weights(packed: torch.Tensor, scales: torch.Tensor, stream=None,
                       deinterleave: bool = False):
    """packed [G, R, K/2], scales [G, R, K/32] (or [R, K/2], [R, K/32]) -> (packed_t, scales_t)
    of the same shapes holding the bytes in the tiled layout of the grouped GEMMs (pass
    MX_WEIGHTS_TILED in the MoE flags to use them). deinterleave: rows alternate gate and up
    (mxfp4_tile_weights_ex with MX_TILE_DEINTERLEAVE)."""
    G = packed.shape[0] if packed.dim() == 3 else 1
    R, K = packed.shape[-2], packed.shape[-1] * 2
    packed_t, scales_t = torch.empty_like(packed), torch.empty_like(scales)
    _check(lib().mxfp4_tile_weights_ex(_ptr(packed), _ptr(scales), G, R, K,
                                       MX_TILE_DEINTERLEAVE if deinterleave else 0, _ptr(packed_t),
                                       _ptr(scales_t), _stream(stream)))
    return packed_t, scales_t


def moe_route_topk(x: torch.Tensor, wr: torch.Tensor, br: torch.Tensor | None, k: int,
                   want_logits: bool = True, stream=None):
    """x [T, H] bf16, wr [E, H] bf16, br [E] fp32 or None -> (logits or None, topk_idx, topk_w).
    want_logits=False passes logits = NULL (the library then selects without storing them)."""
    T, H = x.shape
    E = wr.shape[0]
    dev = x.device
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check(lib().moe_route_topk(_ptr(x), _ptr(wr), _ptr(br), T, H, E, k, _ptr(logits), _ptr(idx),
                                _ptr(w), _stream(stream)))
    return logits, idx, w


def moe_permute(topk_idx: torch.Tensor, E: int, stream=None, use_workspace: bool = True):
    """topk_idx [T, k] int32 -> (offsets [E+1], perm [T*k], inv [T*k]).
    use_workspace: pass moe_permute_workspace bytes (many workgroups for large batches); else
    ws = NULL (one workgroup). Out-of-range indices are reported by get_device_error()."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    nbytes = int(lib().moe_permute_workspace(T, k, E)) if use_workspace else 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    _check(lib().moe_permute(_ptr(topk_idx), T, k, E, _ptr(offsets), _ptr(perm), _ptr(inv),
                             _ptr(ws), nbytes, _stream(stream)))
    return offsets, perm, inv


def get_device_error(stream=None) -> int:
    """mx_get_device_error: synchronizes the stream, returns and clears the device error word of
    the current device (0 = none; MX_DEVERR_ROUTING = a routing index was out of range,
    MX_DEVERR_SYNC = a wait inside a single-launch call gave up)."""
    v = ctypes.c_int32(0)
    _check(lib().mx_get_device_error(_stream(stream), ctypes.byref(v)))
    return int(v.value)


def make_moe_desc(x, gu_packed, gu_scales, dn_packed, dn_scales, k, out, wr=None, br=None,
                  topk_idx=None, topk_w=None, flags=0, topk_idx_out=None, topk_w_out=None,
                  logits_out=None, act=None) -> MoeDesc:
    """act: the expert activation, a dict with any of interleaved (bool), alpha, limit, up_shift
    (floats), gu_bias [E, 2F] and dn_bias [E, H] (fp32 device tensors); None = plain SwiGLU."""
    T, H = x.shape
    E, twoF = gu_packed.shape[0], gu_packed.shape[1]
    d = MoeDesc()
    d.struct_size = ctypes.sizeof(MoeDesc)
    d.T, d.H, d.F, d.E, d.k = T, H, twoF // 2, E, k
    d.flags = flags
    d.out_dtype = _dt(out.dtype)
    d.x, d.wr, d.br = _ptr(x), _ptr(wr), _ptr(br)
    d.topk_idx_in, d.topk_w_in = _ptr(topk_idx), _ptr(topk_w)
    d.gu_packed, d.gu_scales = _ptr(gu_packed), _ptr(gu_scales)
    d.dn_packed, d.dn_scales = _ptr(dn_packed), _ptr(dn_scales)
    d.out = _ptr(out)
    d.topk_idx_out, d.topk_w_out, d.logits_out = (_ptr(topk_idx_out), _ptr(topk_w_out),
                                                   _ptr(logits_out))
    if act:
        d.act_flags = MX_GU_INTERLEAVED if act.get("interleaved") else 0
        d.swiglu_alpha = float(act.get("alpha", 0.0))
        d.swiglu_limit = float(act.get("limit", 0.0))
        d.swiglu_up_shift = float(act.get("up_shift", 0.0))
        d.gu_bias, d.dn_bias = _ptr(act.get("gu_bias")), _ptr(act.get("dn_bias"))
    return d


def mxfp4_moe_mlp_workspace(desc: MoeDesc) -> int:
    return int(lib().mxfp4_moe_mlp_workspace(ctypes.byref(desc)))


def mxfp4_moe_mlp(x, gu_packed, gu_scales, dn_packed, dn_scales, k, wr=None, br=None,
                  topk_idx=None, topk_w=None, out_dtype=torch.bfloat16, flags=0, out=None,
                  workspace=None, return_routing=False, stream=None, act=None):
    """The whole MoE MLP. Weights: gu_packed [E, 2F, H/2], gu_scales [E, 2F, H/32],
    dn_packed [E, H, F/2], dn_scales [E, H, F/32] (with MX_WEIGHTS_TILED in flags: the same
    shapes as written by mxfp4_tile_weights). Routing: internal from (wr, br) unless
    (topk_idx, topk_w) are given. MX_SINGLE_LAUNCH in flags: the whole call as one launch
    (decode-sized batches). Returns out [T, H] (and (logits, idx, w) if asked)."""
    T, H = x.shape
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=dev)
    routing = None
    if return_routing and topk_idx is None:
        E = gu_packed.shape[0]
        routing = (torch.empty((T, E), dtype=torch.float32, device=dev),
                   torch.empty((T, k), dtype=torch.int32, device=dev),
                   torch.empty((T, k), dtype=torch.float32, device=dev))
    d = make_moe_desc(x, gu_packed, gu_scales, dn_packed, dn_scales, k, out, wr=wr, br=br,
                      topk_idx=topk_idx, topk_w=topk_w, flags=flags,
                      topk_idx_out=routing[1] if routing else None,
                      topk_w_out=routing[2] if routing else None,
                      logits_out=routing[0] if routing else None, act=act)
    nbytes = mxfp4_moe_mlp_workspace(d)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _check(lib().mxfp4_moe_mlp(ctypes.byref(d), _ptr(workspace), workspace.numel(),
                               _stream(stream)))
    if return_routing:
        return out, routing
    return out


def mxfp4_moe_mlp_noalloc(desc: MoeDesc, stream=None):
    """mxfp4_moe_mlp_noalloc on a descriptor built by make_moe_desc (its tensors, the output
    included, are the caller's): the workspace is the library's own device array, so neither
    this wrapper nor the library allocates anything."""
    _check(lib().mxfp4_moe_mlp_noalloc(ctypes.byref(desc), _stream(stream)))


def mxfp4_linear_workspace(M: int, K: int, N: int, flags: int = 0) -> int:
    return int(lib().mxfp4_linear_workspace(M, K, N, flags))


def mxfp4_linear(x, packed, scales, out_dtype=torch.float32, flags=0, out=None, workspace=None,
                 stream=None):
    """y [M, N] = x [M, K] (bf16) times the MXFP4 weight [N, K] transposed."""
    M, K = x.shape
    N = packed.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    nbytes = mxfp4_linear_workspace(M, K, N, flags)
    if nbytes and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    _check(lib().mxfp4_linear(_ptr(x), M, K, _ptr(packed), _ptr(scales), N, _ptr(out),
                              _dt(out.dtype), flags, _ptr(workspace) if nbytes else None,
                              nbytes, _stream(stream)))
    return out


def workspace_status(workspace: torch.Tensor, stream=None) -> int:
    v = ctypes.c_int32(0)
    _check(lib().mx_workspace_status(_ptr(workspace), _stream(stream), ctypes.byref(v)))
    return int(v.value)


def version() -> str:
    return lib().mx_version().decode()


def mx_profile_enable(enable: bool = True):
    """Switch per-kernel event timing on or off (clears what was recorded)."""
    _check(lib().mx_profile_enable(1 if enable else 0))


def mx_profile_read() -> dict:
    """{kernel kind: (launches, total milliseconds)} recorded since the last enable/read."""
    buf = (KernelTime * 16)()
    n = lib().mx_profile_read(buf, 16)
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms))
            for i in range(min(n, 16))}
