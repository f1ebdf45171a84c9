"""C-ABI library: it loads, exports every entry point the header declares, and rejects bad
arguments on the host (before touching a device). CPU only: no kernel runs here."""
import ctypes
import re

import pytest
import torch

import mxfp4_weight_quantized_amd as mx


def _declared_functions():
    text = open(mx.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    keep = {n for n in names if n.startswith(("mx", "moe_"))}
    keep -= {"mx_status", "mx_dtype"}
    return sorted(keep)


@pytest.fixture(scope="module")
def L():
    try:
        return mx.lib()
    except RuntimeError as e:
        pytest.fail("HIP library not built: %s" % e)


# The boundary the hot path is specified with: every call, with its parameter list (C types as
# the header spells them, names dropped). mxfp4_linear takes a caller-owned workspace as well
# (the library never allocates; it holds the quantized activations and the split-K partials).
CONTRACT = {
    "mxfp4_quantize": ["const void*", "mx_dtype", "int64_t", "int64_t", "uint8_t*", "uint8_t*",
                       "void*"],
    "mxfp4_dequantize": ["const uint8_t*", "const uint8_t*", "int64_t", "int64_t", "void*",
                         "mx_dtype", "void*"],
    "moe_route_topk": ["const uint16_t*", "const uint16_t*", "const float*", "int32_t", "int32_t",
                       "int32_t", "int32_t", "float*", "int32_t*", "float*", "void*"],
    "moe_permute_workspace": ["int32_t", "int32_t", "int32_t"],
    "moe_permute": ["const int32_t*", "int32_t", "int32_t", "int32_t", "int32_t*", "int32_t*",
                    "int32_t*", "void*", "size_t", "void*"],
    "mxfp4_moe_mlp_workspace": ["const mx_moe_desc*"],
    "mxfp4_moe_mlp": ["const mx_moe_desc*", "void*", "size_t", "void*"],
    "mxfp4_linear": ["const uint16_t*", "int32_t", "int32_t", "const uint8_t*", "const uint8_t*",
                     "int32_t", "void*", "mx_dtype", "uint32_t", "void*", "size_t", "void*"],
    "mx_last_error": [],
    "mx_get_device_error": ["void*", "int32_t*"],
}
# mx_moe_desc fields in order
DESC_FIELDS = ["struct_size", "T", "H", "F", "E", "k", "flags", "out_dtype", "x", "wr", "br",
               "topk_idx_in", "topk_w_in", "gu_packed", "gu_scales", "dn_packed", "dn_scales",
               "out", "topk_idx_out", "topk_w_out", "logits_out"]


def _prototypes():
    """name -> parameter types of every function the header declares."""
    text = re.sub(r"/\*.*?\*/", "", open(mx.HEADER_PATH).read(), flags=re.S)
    protos = {}
    for m in re.finditer(r"\b(?:mx_status|size_t|const char\*|int32_t)\s+([a-z_][a-z0-9_]*)\s*"
                         r"\(([^)]*)\)\s*;", text):
        params = [p.strip() for p in m.group(2).split(",") if p.strip() and p.strip() != "void"]
        types = [re.sub(r"\s*\b[a-zA-Z_][a-zA-Z0-9_]*$", "", p).replace(" *", "*").strip()
                 for p in params]
        protos[m.group(1)] = types
    return protos


def test_header_declares_the_contract():
    protos = _prototypes()
    for name, types in CONTRACT.items():
        assert name in protos, "header does not declare %s" % name
        assert protos[name] == types, (name, protos[name], types)
    fields = [f for f, _ in mx.MoeDesc._fields_]
    assert fields[:len(DESC_FIELDS)] == DESC_FIELDS  # the expert activation fields follow


def test_exports_every_declared_entry_point(L):
    names = _declared_functions()
    assert set(CONTRACT) <= set(names)
    for n in names:
        assert hasattr(L, n), "library does not export %s" % n
    assert set(names) == set(mx.SIGNATURES), "binding signatures out of sync with the header"
    for n, types in _prototypes().items():  # binding arity matches the header
        assert len(mx.SIGNATURES[n][1]) == len(types), n


def test_version_and_error_string(L):
    assert "gfx950" in mx.version()
    assert isinstance(mx.last_error(), str)


def _fake(n=1 << 20):
    # A host address that is never dereferenced: argument checks fail before any launch.
    return ctypes.c_void_p(0x10000000)


def test_quantize_argument_errors(L):
    p = _fake()
    assert L.mxfp4_quantize(p, 7, 4, 64, p, p, None) == mx.MX_ERR_DTYPE
    assert L.mxfp4_quantize(p, mx.MX_F32, 4, 33, p, p, None) == mx.MX_ERR_SHAPE
    assert "multiple of 32" in mx.last_error()
    assert L.mxfp4_quantize(p, mx.MX_F32, -1, 64, p, p, None) == mx.MX_ERR_SHAPE
    assert L.mxfp4_quantize(None, mx.MX_F32, 4, 64, p, p, None) == mx.MX_ERR_NULL
    assert L.mxfp4_quantize(ctypes.c_void_p(0x10000004), mx.MX_F32, 4, 64, p, p, None) == mx.MX_ERR_ALIGN
    assert L.mxfp4_quantize(p, mx.MX_F32, 0, 64, p, p, None) == mx.MX_OK  # empty: no-op
    assert L.mxfp4_dequantize(p, p, 4, 48, p, mx.MX_F32, None) == mx.MX_ERR_SHAPE
    assert L.mxfp4_dequantize(p, p, 4, 64, p, 9, None) == mx.MX_ERR_DTYPE
    assert L.mxfp4_dequantize(p, p, 0, 64, p, mx.MX_BF16, None) == mx.MX_OK


def test_tile_weights_argument_errors(L):
    p = _fake()
    assert L.mxfp4_tile_weights(p, p, 2, 24, 64, p, p, None) == mx.MX_ERR_SHAPE  # R % 16
    assert L.mxfp4_tile_weights(p, p, 2, 32, 48, p, p, None) == mx.MX_ERR_SHAPE  # K % 32
    assert L.mxfp4_tile_weights(p, p, -1, 32, 64, p, p, None) == mx.MX_ERR_SHAPE
    assert L.mxfp4_tile_weights(p, None, 2, 32, 64, p, p, None) == mx.MX_ERR_NULL
    assert L.mxfp4_tile_weights(p, p, 2, 32, 64, p, None, None) == mx.MX_ERR_NULL
    assert L.mxfp4_tile_weights(ctypes.c_void_p(0x10000008), p, 2, 32, 64, p, p, None) == mx.MX_ERR_ALIGN
    assert L.mxfp4_tile_weights(p, p, 0, 32, 64, p, p, None) == mx.MX_OK  # empty: no-op
    assert L.mxfp4_tile_weights_ex(p, p, 2, 48, 64, 1, p, p, None) == mx.MX_ERR_SHAPE  # R % 32
    assert L.mxfp4_tile_weights_ex(p, p, 2, 64, 64, 2, p, p, None) == mx.MX_ERR_UNSUPPORTED
    assert L.mxfp4_tile_weights_ex(p, p, 0, 64, 64, 1, p, p, None) == mx.MX_OK


def test_route_and_permute_argument_errors(L):
    p = _fake()
    assert L.moe_route_topk(p, p, None, 4, 64, 8, 9, p, p, p, None) == mx.MX_ERR_SHAPE  # k > E
    assert L.moe_route_topk(p, p, None, 4, 64, 300, 4, p, p, p, None) == mx.MX_ERR_SHAPE  # E > 256
    assert L.moe_route_topk(p, p, None, 4, 64, 32, 9, p, p, p, None) == mx.MX_ERR_SHAPE  # k > 8
    assert L.moe_route_topk(p, p, None, 4, 48, 32, 4, p, p, p, None) == mx.MX_ERR_SHAPE  # H % 32
    assert L.moe_route_topk(p, None, None, 4, 64, 32, 4, p, p, p, None) == mx.MX_ERR_NULL
    assert L.moe_route_topk(p, p, None, 4, 64, 32, 4, None, None, p, None) == mx.MX_ERR_NULL  # idx
    assert L.moe_route_topk(p, p, None, 0, 64, 32, 4, p, p, p, None) == mx.MX_OK  # T = 0
    assert L.moe_route_topk(p, p, None, 0, 64, 32, 4, None, p, p, None) == mx.MX_OK  # no logits
    assert L.moe_permute(p, 4, 2, 8, None, p, p, None, 0, None) == mx.MX_ERR_NULL
    need = mx.lib().moe_permute_workspace(4096, 4, 32)  # 16 384 pairs: the sliced path
    assert need > 0 and need % 256 == 0 and mx.lib().moe_permute_workspace(64, 4, 32) == 0
    assert L.moe_permute(p, 4096, 4, 32, p, p, p, p, need - 1, None) == mx.MX_ERR_WORKSPACE
    assert L.moe_permute(p, 4096, 4, 32, p, p, p, ctypes.c_void_p(0x10000010), need,
                         None) == mx.MX_ERR_ALIGN
    assert L.moe_permute(p, 4, 9, 8, p, p, p, None, 0, None) == mx.MX_ERR_SHAPE
    assert L.moe_permute(p, 4, 0, 8, p, p, p, None, 0, None) == mx.MX_ERR_SHAPE
    assert L.mx_get_device_error(None, None) == mx.MX_ERR_NULL


def _desc(T=4, H=64, F=64, E=8, k=2, **kw):
    d = mx.MoeDesc()
    d.struct_size = ctypes.sizeof(mx.MoeDesc)
    d.T, d.H, d.F, d.E, d.k = T, H, F, E, k
    d.out_dtype = mx.MX_F32
    p = 0x10000000
    for f in ("x", "wr", "gu_packed", "gu_scales", "dn_packed", "dn_scales", "out"):
        setattr(d, f, p)
    for f, v in kw.items():
        setattr(d, f, v)
    return d


def test_moe_workspace_query_and_errors(L):
    d = _desc(T=64, H=2880, F=2880, E=32, k=4)
    n = mx.mxfp4_moe_mlp_workspace(d)
    P = 64 * 4
    # at least the bf16 SwiGLU output and the fp32 per-pair expert outputs
    assert n >= P * 2880 * 2 + P * 2880 * 4 and n % 256 == 0
    d_mx = _desc(T=64, H=2880, F=2880, E=32, k=4, flags=mx.MX_ACT_MXFP4)
    # the activation variant keeps no bf16 h (gate_up writes it as MXFP4): smaller, still the
    # fp32 per-pair rows and the packed h
    n_mx = mx.mxfp4_moe_mlp_workspace(d_mx)
    assert P * 2880 * 4 + P * 2880 * 17 // 32 <= n_mx < n
    bad = _desc()
    bad.struct_size = 8
    assert mx.mxfp4_moe_mlp_workspace(bad) == 0
    assert L.mxfp4_moe_mlp(ctypes.byref(bad), _fake(), 1 << 30, None) == mx.MX_ERR_UNSUPPORTED
    assert L.mxfp4_moe_mlp(None, _fake(), 1 << 30, None) == mx.MX_ERR_NULL
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(H=48)), _fake(), 1 << 30, None) == mx.MX_ERR_SHAPE
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(k=9)), _fake(), 1 << 30, None) == mx.MX_ERR_SHAPE
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(flags=8)), _fake(), 1 << 30, None) == mx.MX_ERR_UNSUPPORTED
    for fl in (mx.MX_WEIGHTS_TILED, mx.MX_WEIGHTS_TILED | mx.MX_ACT_MXFP4, mx.MX_SINGLE_LAUNCH,
               mx.MX_SINGLE_LAUNCH | mx.MX_WEIGHTS_TILED):  # accepted flags
        assert L.mxfp4_moe_mlp(ctypes.byref(_desc(flags=fl, x=0)), _fake(), 1 << 30,
                               None) == mx.MX_ERR_NULL
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(out_dtype=5)), _fake(), 1 << 30, None) == mx.MX_ERR_DTYPE
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(x=0)), _fake(), 1 << 30, None) == mx.MX_ERR_NULL
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(x=0x10000002)), _fake(), 1 << 30, None) == mx.MX_ERR_ALIGN
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(wr=0)), _fake(), 1 << 30, None) == mx.MX_ERR_NULL
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(topk_idx_in=0x10000000)), _fake(), 1 << 30,
                           None) == mx.MX_ERR_NULL  # weights missing
    small = _desc()
    need = mx.mxfp4_moe_mlp_workspace(small)
    assert L.mxfp4_moe_mlp(ctypes.byref(small), _fake(), need - 1, None) == mx.MX_ERR_WORKSPACE
    assert L.mxfp4_moe_mlp(ctypes.byref(small), None, need, None) == mx.MX_ERR_WORKSPACE
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(T=0)), None, 0, None) == mx.MX_OK
    # the descriptor without the expert activation fields is accepted (they read as zero)
    v1 = mx.MoeDesc.act_flags.offset
    old_desc = _desc(T=64, H=2880, F=2880, E=32, k=4, struct_size=v1)
    assert mx.mxfp4_moe_mlp_workspace(old_desc) == n
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(struct_size=v1, x=0)), _fake(), 1 << 30,
                           None) == mx.MX_ERR_NULL
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(struct_size=v1 + 4)), _fake(), 1 << 30,
                           None) == mx.MX_ERR_UNSUPPORTED
    # interleaved gate/up rows need the tiled layout; unknown activation flags; non-finite params
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(act_flags=mx.MX_GU_INTERLEAVED)), _fake(), 1 << 30,
                           None) == mx.MX_ERR_UNSUPPORTED
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(act_flags=4)), _fake(), 1 << 30,
                           None) == mx.MX_ERR_UNSUPPORTED
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(swiglu_limit=float("inf"))), _fake(), 1 << 30,
                           None) == mx.MX_ERR_SHAPE
    # the single launch: decode-sized batches of bf16 activations only; its workspace adds the
    # partial router logits and drops the sliced permutation's counts
    S = mx.MX_SINGLE_LAUNCH
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(flags=S | mx.MX_ACT_MXFP4)), _fake(), 1 << 30,
                           None) == mx.MX_ERR_UNSUPPORTED
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(T=513, k=4, flags=S)), _fake(), 1 << 30,
                           None) == mx.MX_ERR_UNSUPPORTED
    assert "decode-sized" in mx.last_error()
    assert L.mxfp4_moe_mlp(ctypes.byref(_desc(T=512, k=4, flags=S, x=0)), _fake(), 1 << 30,
                           None) == mx.MX_ERR_NULL
    n_single = mx.mxfp4_moe_mlp_workspace(_desc(T=64, H=2880, F=2880, E=32, k=4, flags=S))
    assert n < n_single <= n + 8 * 64 * 32 * 4 + 2 * 256
    # the allocation-free entry point: same checks, and problems beyond its array are rejected
    # on the host before anything runs
    big = _desc(T=8192, H=2880, F=2880, E=32, k=4)
    assert mx.mxfp4_moe_mlp_workspace(big) > mx.MX_NOALLOC_SCRATCH_BYTES
    assert L.mxfp4_moe_mlp_noalloc(ctypes.byref(big), None) == mx.MX_ERR_WORKSPACE
    assert "allocation-free" in mx.last_error()
    assert L.mxfp4_moe_mlp_noalloc(ctypes.byref(_desc(k=9)), None) == mx.MX_ERR_SHAPE
    assert L.mxfp4_moe_mlp_noalloc(None, None) == mx.MX_ERR_NULL
    assert L.mxfp4_moe_mlp_noalloc(ctypes.byref(_desc(T=0)), None) == mx.MX_OK


def test_linear_argument_errors(L):
    p = _fake()
    assert L.mxfp4_linear(p, 4, 40, p, p, 8, p, mx.MX_F32, 0, None, 0, None) == mx.MX_ERR_SHAPE
    assert L.mxfp4_linear(p, 4, 64, p, p, 8, p, 3, 0, None, 0, None) == mx.MX_ERR_DTYPE
    assert L.mxfp4_linear(p, 4, 16384, p, p, 8, p, mx.MX_F32, 0, None, 0, None) == mx.MX_ERR_SHAPE
    assert L.mxfp4_linear(p, 4, 64, p, p, 8, p, mx.MX_F32, 2, None, 0, None) == mx.MX_ERR_UNSUPPORTED
    assert L.mxfp4_linear(None, 4, 64, p, p, 8, p, mx.MX_F32, 0, None, 0, None) == mx.MX_ERR_NULL
    assert L.mxfp4_linear(p, 0, 64, p, p, 8, p, mx.MX_F32, 0, None, 0, None) == mx.MX_OK
    assert mx.mxfp4_linear_workspace(4, 64, 8, 0) == 0
    assert mx.mxfp4_linear_workspace(4, 64, 8, mx.MX_ACT_MXFP4) > 0
    assert L.mxfp4_linear(p, 4, 64, p, p, 8, p, mx.MX_F32, mx.MX_ACT_MXFP4, None, 0,
                          None) == mx.MX_ERR_WORKSPACE
    # decode-sized M splits K: the partial sums need a workspace even for bf16 activations
    need = mx.mxfp4_linear_workspace(1, 2880, 5760, 0)
    assert need >= 2 * 1 * 5760 * 4 and need % 256 == 0
    assert mx.mxfp4_linear_workspace(1, 2880, 5760, mx.MX_ACT_MXFP4) > need
    assert mx.mxfp4_linear_workspace(128, 2880, 5760, 0) == 0  # prefill-sized: no split
    assert L.mxfp4_linear(p, 1, 2880, p, p, 5760, p, mx.MX_BF16, 0, None, 0,
                          None) == mx.MX_ERR_WORKSPACE
    assert L.mxfp4_linear(p, 1, 2880, p, p, 5760, p, mx.MX_BF16, 0, p, need - 1,
                          None) == mx.MX_ERR_WORKSPACE


def test_binding_rejects_cpu_tensors():
    x = torch.zeros(4, 64, dtype=torch.float32)
    with pytest.raises(ValueError):
        mx.mxfp4_quantize(x)
