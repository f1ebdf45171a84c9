// abi.hip -- the C ABI (include/mxfp4moe.h): host-side argument checks, workspace layout and the
// launch sequence. No allocation, no synchronization (except mx_workspace_status), no C++
// exception crosses the boundary.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/mxfp4moe.h"
#include "mx_launch.h"

#define MX_API extern "C" __attribute__((visibility("default")))
static_assert(MX_MAX_TOPK <= 8 && MX_MAX_MOE_DIM <= 3072, "combine launch: k <= 8, H / 8 <= 384 threads");

namespace {

thread_local char g_err[512] = "";

mx_status fail(mx_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

mx_status ok() {
  g_err[0] = 0;
  return MX_OK;
}

mx_status hip_fail(hipError_t e, const char* what) {
  return fail(MX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

// gfx950 check for the current device (cached per device).
mx_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MX_ERR_UNSUPPORTED, "device index %d", dev);
  int v = g_arch_ok[dev].load(std::memory_order_acquire);
  if (v == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    v = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(v, std::memory_order_release);
  }
  if (v != 1) return fail(MX_ERR_UNSUPPORTED, "this library runs on gfx950 (MI355X) devices only");
  return MX_OK;
}

// ---- opt-in per-kernel timing (benchmarks): HIP events on the caller's stream ----
enum ProfKind { PK_QUANTIZE, PK_DEQUANTIZE, PK_ROUTE, PK_PERMUTE, PK_GATE_UP, PK_DOWN, PK_COMBINE,
                PK_LINEAR, PK_TILE, PK_SINGLE, PK_COUNT };
const char* const kProfNames[PK_COUNT] = {"quantize", "dequantize", "route_topk", "permute",
                                          "moe_gate_up_swiglu", "moe_down_weighted", "moe_combine",
                                          "linear", "tile_weights", "moe_single_launch"};
struct ProfRec {
  int kind;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t prof_event() {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  // timing only: no system-scope fence when the event is recorded (a cache write-back and
  // invalidation that lengthened every bracketed decode-sized kernel by a few us)
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Brackets one kernel launch with two events when profiling is on; no-op otherwise.
struct ProfScope {
  int kind;
  hipStream_t s;
  hipEvent_t a = nullptr;
  ProfScope(int k, hipStream_t st) : kind(k), s(st) {
    if (g_prof_on.load(std::memory_order_relaxed)) {
      a = prof_event();
      if (a) hipEventRecord(a, s);
    }
  }
  ~ProfScope() {
    if (!a) return;
    hipEvent_t b = prof_event();
    if (!b) return;
    hipEventRecord(b, s);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_recs.push_back({kind, a, b});
  }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// ---- mxfp4_moe_mlp workspace layout ----
struct MoeLayout {
  size_t status, logits, idx, w, offsets, perm, inv, tiles, pcounts, rpart, tile_ends, h, y, xq, xq_tok, xqs_tok, xqs,
      hq, hqs,
      total;
  size_t pcounts_bytes;
  int tile_rows, max_tiles;
};

MoeLayout moe_layout(const mx_moe_desc& d) {
  MoeLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t T = (size_t)d.T, P = (size_t)d.T * d.k, E = (size_t)d.E;
  const bool single = (d.flags & MX_SINGLE_LAUNCH) != 0;
  L.tile_rows = single ? 16 : mx::moe_tile_rows(d.T, d.k, d.E, (d.flags & MX_ACT_MXFP4) != 0);
  L.max_tiles = mx::moe_max_tiles(d.T, d.k, d.E, L.tile_rows);
  L.status = take(256);  // int32 status, int32 tile count, int32 counter of the routing launch
  L.logits = take(T * E * 4);
  L.idx = take(P * 4);
  L.w = take(P * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take((P + mx::kMaxTileRows) * 4);  // tile-row padding (see launch_permute)
  L.inv = take(P * 4);
  L.tiles = take((size_t)L.max_tiles * 8);
  L.pcounts_bytes = single ? 0 : mx::permute_sliced_workspace(d.T, d.k, d.E);  // 0: one workgroup
  L.pcounts = take(L.pcounts_bytes);
  // the single launch's partial router logits (the split launches borrow y's rows for theirs)
  L.rpart = single ? take((size_t)mx::single_route_splits(d.T, d.H, d.E) * T * E * 4) : 0;
  L.tile_ends = single ? take((size_t)L.max_tiles * 4) : 0;
  // bf16 h (the activation variant quantizes h in the gate_up epilogue and keeps only hq, hqs)
  L.h = (d.flags & MX_ACT_MXFP4) ? 0 : take(P * (size_t)d.F * 2);
  L.y = take(P * (size_t)d.H * 4);
  if (d.flags & MX_ACT_MXFP4) {
    // scales block-major in pair order; codes: prefill-shaped calls take x in token order, then
    // x and h in pair order tiled by 16 rows ([P/16][K/32][16][16]); decode-shaped calls x in
    // token order and h in pair order, row-major
    const bool pre = L.tile_rows != 16;
    const size_t P16 = (P + 15) / 16 * 16;
    L.xq = take((pre ? P16 : T) * (size_t)d.H / 2);
    L.xq_tok = pre ? take(T * (size_t)d.H / 2) : 0;
    L.xqs_tok = pre ? take(T * (size_t)d.H / 32) : 0;
    L.xqs = take((P + 3) / 4 * 4 * (size_t)d.H / 32);  // block-major [H/32][P rounded up to 4]
    L.hq = take((pre ? P16 : P) * (size_t)d.F / 2);
    L.hqs = take((P + 3) / 4 * 4 * (size_t)d.F / 32);  // block-major [F/32][P rounded up to 4]
  }
  L.total = off;
  return L;
}

mx_status check_routing_shape(int64_t T, int64_t H, int64_t E, int64_t k) {
  if (T < 0 || H <= 0 || E <= 0 || k <= 0) return fail(MX_ERR_SHAPE, "T=%lld H=%lld E=%lld k=%lld", (long long)T, (long long)H, (long long)E, (long long)k);
  if (E > MX_MAX_EXPERTS) return fail(MX_ERR_SHAPE, "E=%lld exceeds %d", (long long)E, MX_MAX_EXPERTS);
  if (k > E || k > MX_MAX_TOPK) return fail(MX_ERR_SHAPE, "k=%lld must be <= min(E, %d)", (long long)k, MX_MAX_TOPK);
  if (T * k >= (1LL << 31)) return fail(MX_ERR_SHAPE, "T*k too large");
  return MX_OK;
}

// The caller's descriptor as the current version: one that ends at logits_out (the size before
// the expert activation fields) reads those fields as zero.
mx_status read_desc(const mx_moe_desc* in, mx_moe_desc* out) {
  if (in == nullptr) return fail(MX_ERR_NULL, "desc is NULL");
  if (in->struct_size == sizeof(mx_moe_desc)) {
    *out = *in;
  } else if (in->struct_size == MX_MOE_DESC_SIZE_V1) {
    std::memset(out, 0, sizeof(*out));
    std::memcpy(out, in, MX_MOE_DESC_SIZE_V1);
  } else {
    return fail(MX_ERR_UNSUPPORTED, "desc.struct_size %zu (expected %zu or %zu)", in->struct_size,
                sizeof(mx_moe_desc), (size_t)MX_MOE_DESC_SIZE_V1);
  }
  return MX_OK;
}

bool act_custom(const mx_moe_desc& d) {
  return d.act_flags != 0 || d.swiglu_alpha != 0.f || d.swiglu_limit > 0.f ||
         d.swiglu_up_shift != 0.f || d.gu_bias != nullptr || d.dn_bias != nullptr;
}

mx_status check_moe_desc(const mx_moe_desc* d) {
  if (d == nullptr) return fail(MX_ERR_NULL, "desc is NULL");
  mx_status st = check_routing_shape(d->T, d->H, d->E, d->k);
  if (st != MX_OK) return st;
  if (d->F <= 0 || d->H % 32 || d->F % 32) return fail(MX_ERR_SHAPE, "H=%d and F=%d must be positive multiples of 32", d->H, d->F);
  if (d->H > MX_MAX_MOE_DIM || d->F > MX_MAX_MOE_DIM) return fail(MX_ERR_SHAPE, "H and F must be <= %d in the MoE MLP", MX_MAX_MOE_DIM);
  if ((int64_t)d->T * d->H * 2 >= (1LL << 31) || (int64_t)d->T * d->k * d->F * 2 >= (1LL << 31))
    return fail(MX_ERR_SHAPE, "T*H and T*k*F bf16 activations must stay below 2 GiB");
  if (d->flags & ~(MX_ACT_MXFP4 | MX_WEIGHTS_TILED | MX_SINGLE_LAUNCH)) return fail(MX_ERR_UNSUPPORTED, "unknown flags 0x%x", d->flags);
  if ((d->flags & MX_SINGLE_LAUNCH) && (d->flags & MX_ACT_MXFP4))
    return fail(MX_ERR_UNSUPPORTED, "MX_SINGLE_LAUNCH takes bf16 activations (not with MX_ACT_MXFP4)");
  if ((d->flags & MX_SINGLE_LAUNCH) && (int64_t)d->T * d->k > mx::kSingleMaxPairs)
    return fail(MX_ERR_UNSUPPORTED, "MX_SINGLE_LAUNCH takes decode-sized batches: T*k = %lld > %d",
                (long long)d->T * d->k, mx::kSingleMaxPairs);
  if (d->act_flags & ~MX_GU_INTERLEAVED) return fail(MX_ERR_UNSUPPORTED, "unknown act_flags 0x%x", d->act_flags);
  if ((d->act_flags & MX_GU_INTERLEAVED) && !(d->flags & MX_WEIGHTS_TILED))
    return fail(MX_ERR_UNSUPPORTED, "interleaved gate/up rows need the tiled layout "
                "(mxfp4_tile_weights_ex with MX_TILE_DEINTERLEAVE, flag MX_WEIGHTS_TILED)");
  if ((d->gu_bias && !aligned(d->gu_bias, 4)) || (d->dn_bias && !aligned(d->dn_bias, 16)))
    return fail(MX_ERR_ALIGN, "gu_bias must be 4-byte and dn_bias 16-byte aligned");
  if (!std::isfinite(d->swiglu_alpha) || !std::isfinite(d->swiglu_limit) || !std::isfinite(d->swiglu_up_shift))
    return fail(MX_ERR_SHAPE, "swiglu_alpha, swiglu_limit and swiglu_up_shift must be finite");
  if (d->out_dtype != MX_F32 && d->out_dtype != MX_BF16) return fail(MX_ERR_DTYPE, "out_dtype %d", (int)d->out_dtype);
  if (d->T == 0) return MX_OK;
  if (!d->x || !d->gu_packed || !d->gu_scales || !d->dn_packed || !d->dn_scales || !d->out)
    return fail(MX_ERR_NULL, "x, weights, scales and out are required");
  if (d->topk_idx_in == nullptr && d->wr == nullptr) return fail(MX_ERR_NULL, "wr is required for internal routing");
  if (d->topk_idx_in != nullptr && d->topk_w_in == nullptr) return fail(MX_ERR_NULL, "topk_w_in is required with topk_idx_in");
  const void* a16[] = {d->x, d->wr, d->gu_packed, d->gu_scales, d->dn_packed, d->dn_scales, d->out};
  for (const void* p : a16)
    if (p && !aligned(p, 16)) return fail(MX_ERR_ALIGN, "x, wr, weights, scales and out must be 16-byte aligned");
  return MX_OK;
}

}  // namespace

// =============================================================================================
MX_API mx_status mxfp4_quantize(const void* src, mx_dtype src_dtype, int64_t rows, int64_t K,
                                uint8_t* packed, uint8_t* scales, void* stream) {
  if (src_dtype != MX_F32 && src_dtype != MX_BF16) return fail(MX_ERR_DTYPE, "src_dtype %d", (int)src_dtype);
  if (rows < 0 || K < 0 || K % 32) return fail(MX_ERR_SHAPE, "rows=%lld K=%lld (K must be a multiple of 32)", (long long)rows, (long long)K);
  if (rows == 0 || K == 0) return ok();
  if (!src || !packed || !scales) return fail(MX_ERR_NULL, "src, packed and scales are required");
  if (!aligned(src, src_dtype == MX_F32 ? 16 : 8) || !aligned(packed, 16)) return fail(MX_ERR_ALIGN, "src or packed misaligned");
  mx_status st = check_device();
  if (st != MX_OK) return st;
  ProfScope ps(PK_QUANTIZE, (hipStream_t)stream);
  hipError_t e = mx::launch_quantize(src, src_dtype == MX_BF16, rows * (K / 32), packed, scales, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "quantize launch");
}

MX_API mx_status mxfp4_dequantize(const uint8_t* packed, const uint8_t* scales, int64_t rows,
                                  int64_t K, void* dst, mx_dtype dst_dtype, void* stream) {
  if (dst_dtype != MX_F32 && dst_dtype != MX_BF16) return fail(MX_ERR_DTYPE, "dst_dtype %d", (int)dst_dtype);
  if (rows < 0 || K < 0 || K % 32) return fail(MX_ERR_SHAPE, "rows=%lld K=%lld (K must be a multiple of 32)", (long long)rows, (long long)K);
  if (rows == 0 || K == 0) return ok();
  if (!packed || !scales || !dst) return fail(MX_ERR_NULL, "packed, scales and dst are required");
  if (!aligned(packed, 16) || !aligned(dst, 16)) return fail(MX_ERR_ALIGN, "packed or dst misaligned");
  mx_status st = check_device();
  if (st != MX_OK) return st;
  ProfScope ps(PK_DEQUANTIZE, (hipStream_t)stream);
  hipError_t e = mx::launch_dequantize(packed, scales, rows * (K / 32), dst, dst_dtype == MX_BF16, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "dequantize launch");
}

MX_API mx_status mxfp4_tile_weights(const uint8_t* packed, const uint8_t* scales, int64_t G,
                                    int64_t R, int64_t K, uint8_t* packed_t, uint8_t* scales_t,
                                    void* stream) {
  return mxfp4_tile_weights_ex(packed, scales, G, R, K, 0u, packed_t, scales_t, stream);
}

MX_API mx_status mxfp4_tile_weights_ex(const uint8_t* packed, const uint8_t* scales, int64_t G,
                                       int64_t R, int64_t K, uint32_t flags, uint8_t* packed_t,
                                       uint8_t* scales_t, void* stream) {
  if (flags & ~MX_TILE_DEINTERLEAVE) return fail(MX_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  if ((flags & MX_TILE_DEINTERLEAVE) && R % 32)
    return fail(MX_ERR_SHAPE, "R=%lld: de-interleaving needs R a multiple of 32", (long long)R);
  if (G < 0 || R < 0 || K < 0 || R % 16 || K % 32 || R > INT32_MAX || K > INT32_MAX)
    return fail(MX_ERR_SHAPE, "G=%lld R=%lld K=%lld (R a multiple of 16, K of 32)", (long long)G,
                (long long)R, (long long)K);
  if (G == 0 || R == 0 || K == 0) return ok();
  if (!packed || !scales || !packed_t || !scales_t) return fail(MX_ERR_NULL, "packed, scales, packed_t and scales_t are required");
  if (!aligned(packed, 16) || !aligned(packed_t, 16)) return fail(MX_ERR_ALIGN, "packed and packed_t must be 16-byte aligned");
  mx_status st = check_device();
  if (st != MX_OK) return st;
  ProfScope ps(PK_TILE, (hipStream_t)stream);
  hipError_t e = mx::launch_tile_weights(packed, scales, G, (int)R, (int)K,
                                         (flags & MX_TILE_DEINTERLEAVE) != 0, packed_t, scales_t,
                                         (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "tile_weights launch");
}

MX_API mx_status moe_route_topk(const uint16_t* x, const uint16_t* wr, const float* br, int32_t T,
                                int32_t H, int32_t E, int32_t k, float* logits, int32_t* topk_idx,
                                float* topk_w, void* stream) {
  mx_status st = check_routing_shape(T, H, E, k);
  if (st != MX_OK) return st;
  if (H % 32) return fail(MX_ERR_SHAPE, "H=%d must be a multiple of 32", H);
  if (T == 0) return ok();
  if (!x || !wr || !topk_idx || !topk_w)
    return fail(MX_ERR_NULL, "x, wr, topk_idx and topk_w are required");
  if (!aligned(x, 16) || !aligned(wr, 16)) return fail(MX_ERR_ALIGN, "x and wr must be 16-byte aligned");
  st = check_device();
  if (st != MX_OK) return st;
  ProfScope ps(PK_ROUTE, (hipStream_t)stream);
  hipError_t e = mx::launch_route_topk(x, wr, br, T, H, E, k, logits, topk_idx, topk_w, nullptr, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "route launch");
}

MX_API size_t moe_permute_workspace(int32_t T, int32_t k, int32_t E) {
  if (check_routing_shape(T, 32, E, k) != MX_OK) return 0;
  return align256(mx::permute_sliced_workspace(T, k, E));
}

MX_API mx_status moe_permute(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                             int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                             size_t ws_bytes, void* stream) {
  mx_status st = check_routing_shape(T, 32, E, k);
  if (st != MX_OK) return st;
  if (!offsets) return fail(MX_ERR_NULL, "offsets is required");
  if (T > 0 && (!topk_idx || !perm || !inv)) return fail(MX_ERR_NULL, "topk_idx, perm and inv are required");
  const size_t need = align256(mx::permute_sliced_workspace(T, k, E));  // as moe_permute_workspace
  const bool sliced = need > 0 && ws != nullptr;  // ws NULL: one workgroup does it all
  if (sliced && ws_bytes < need) return fail(MX_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (sliced && !aligned(ws, 256)) return fail(MX_ERR_ALIGN, "workspace must be 256-byte aligned");
  st = check_device();
  if (st != MX_OK) return st;
  ProfScope ps(PK_PERMUTE, (hipStream_t)stream);
  hipError_t e = sliced
      ? mx::launch_permute_sliced(topk_idx, T, k, E, offsets, perm, inv, nullptr, 0, nullptr,
                                  nullptr, static_cast<int32_t*>(ws), (hipStream_t)stream)
      : mx::launch_permute(topk_idx, T, k, E, offsets, perm, inv, nullptr, 0, nullptr, nullptr,
                           (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "permute launch");
}

MX_API size_t mxfp4_moe_mlp_workspace(const mx_moe_desc* desc) {
  mx_moe_desc d;
  if (read_desc(desc, &d) != MX_OK) return 0;
  if (check_routing_shape(d.T, d.H, d.E, d.k) != MX_OK || d.F <= 0) return 0;
  return moe_layout(d).total;
}

namespace {
// The launch sequence of mxfp4_moe_mlp on a checked descriptor, its layout and a workspace of at
// least L.total bytes (256-byte aligned).
mx_status moe_mlp_run(const mx_moe_desc& d, const MoeLayout& L, char* w, hipStream_t s);
}  // namespace

MX_API mx_status mxfp4_moe_mlp(const mx_moe_desc* desc, void* ws, size_t ws_bytes, void* stream) {
  mx_moe_desc d;
  mx_status st = read_desc(desc, &d);
  if (st != MX_OK) return st;
  st = check_moe_desc(&d);
  if (st != MX_OK) return st;
  if (d.T == 0) return ok();
  const MoeLayout L = moe_layout(d);
  if (ws == nullptr || ws_bytes < L.total) return fail(MX_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", L.total, ws_bytes);
  if (!aligned(ws, 256)) return fail(MX_ERR_ALIGN, "workspace must be 256-byte aligned");
  st = check_device();
  if (st != MX_OK) return st;
  return moe_mlp_run(d, L, static_cast<char*>(ws), (hipStream_t)stream);
}

// ---- the allocation-free variant: the workspace is the library's own device array ----
// One array per device (each GPU the library runs on holds its own copy at its own address, until
// the process ends). Host code never passes `scratch` itself -- on the host that name is only a
// stand-in -- but the device address hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) uint8_t scratch[MX_NOALLOC_SCRATCH_BYTES];

namespace {
std::atomic<char*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (nullptr and an error message on failure).
char* scratch_on_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  char* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* a = nullptr;
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess || a == nullptr) {
      hip_fail(e, "scratch lookup");
      return nullptr;
    }
    p = static_cast<char*>(a);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}
}  // namespace

MX_API mx_status mxfp4_moe_mlp_noalloc(const mx_moe_desc* desc, void* stream) {
  mx_moe_desc d;
  mx_status st = read_desc(desc, &d);
  if (st != MX_OK) return st;
  st = check_moe_desc(&d);
  if (st != MX_OK) return st;
  if (d.T == 0) return ok();
  const MoeLayout L = moe_layout(d);
  if (L.total > (size_t)MX_NOALLOC_SCRATCH_BYTES)
    return fail(MX_ERR_WORKSPACE, "this problem needs %zu bytes of workspace; the allocation-free "
                "entry point holds %zu (use mxfp4_moe_mlp with a caller workspace)",
                L.total, (size_t)MX_NOALLOC_SCRATCH_BYTES);
  st = check_device();
  if (st != MX_OK) return st;
  char* w = scratch_on_device();
  if (w == nullptr) return MX_ERR_HIP;
  return moe_mlp_run(d, L, w, (hipStream_t)stream);
}

namespace {
// The GEMM-side arguments of a call (routing outputs in the workspace unless the caller asked
// for them or gave its own routing).
mx::MoeGemmArgs gemm_args(const mx_moe_desc& d, const MoeLayout& L, char* w, const int32_t* idx,
                          const float* tw) {
  const bool mx_act = (d.flags & MX_ACT_MXFP4) != 0;
  mx::MoeGemmArgs g{};
  g.T = d.T; g.H = d.H; g.F = d.F; g.E = d.E; g.k = d.k;
  g.mx_act = mx_act;
  g.tiled = (d.flags & MX_WEIGHTS_TILED) != 0;
  g.xq = reinterpret_cast<uint8_t*>(w + L.xq);
  g.xqs = reinterpret_cast<uint8_t*>(w + L.xqs);
  g.hq = reinterpret_cast<uint8_t*>(w + L.hq);
  g.hqs = reinterpret_cast<uint8_t*>(w + L.hqs);
  g.hqs_pitch = ((int64_t)d.T * d.k + 3) / 4 * 4;
  g.x = d.x;
  g.perm = reinterpret_cast<int32_t*>(w + L.perm);
  g.inv = reinterpret_cast<int32_t*>(w + L.inv);
  g.offsets = reinterpret_cast<int32_t*>(w + L.offsets);
  g.tiles = reinterpret_cast<int2*>(w + L.tiles);
  g.num_tiles = reinterpret_cast<int32_t*>(w + L.status) + 1;
  g.max_tiles = L.max_tiles;
  g.topk_w = tw;
  g.topk_idx = idx;
  g.gu_packed = d.gu_packed; g.gu_scales = d.gu_scales;
  g.dn_packed = d.dn_packed; g.dn_scales = d.dn_scales;
  g.h = mx_act ? nullptr : reinterpret_cast<uint16_t*>(w + L.h);
  g.y = reinterpret_cast<float*>(w + L.y);
  g.out = d.out;
  g.out_bf16 = d.out_dtype == MX_BF16;
  if (act_custom(d)) {
    g.act_custom = true;
    g.gu_bias = d.gu_bias;
    g.dn_bias = d.dn_bias;
    g.gu_interleaved = (d.act_flags & MX_GU_INTERLEAVED) != 0;
    g.act_alpha = d.swiglu_alpha != 0.f ? d.swiglu_alpha : 1.f;
    g.act_limit = d.swiglu_limit;
    g.act_shift = d.swiglu_up_shift;
  }
  return g;
}

// MX_SINGLE_LAUNCH: everything in one launch.
mx_status moe_mlp_single(const mx_moe_desc& d, const MoeLayout& L, char* w, hipStream_t s) {
  const bool route = d.topk_idx_in == nullptr;
  const int32_t* idx = route ? (d.topk_idx_out ? d.topk_idx_out : reinterpret_cast<int32_t*>(w + L.idx))
                             : d.topk_idx_in;
  const float* tw = route ? (d.topk_w_out ? d.topk_w_out : reinterpret_cast<float*>(w + L.w))
                          : d.topk_w_in;
  const mx::MoeGemmArgs g = gemm_args(d, L, w, idx, tw);
  mx::SingleRouting r{};
  r.wr = route ? d.wr : nullptr;
  r.br = d.br;
  r.logits = route ? d.logits_out : nullptr;
  r.rpart = reinterpret_cast<float*>(w + L.rpart);
  r.tile_ends = reinterpret_cast<int32_t*>(w + L.tile_ends);
  r.status = reinterpret_cast<int32_t*>(w + L.status);
  ProfScope ps(PK_SINGLE, s);
  const hipError_t e = mx::launch_moe_single(g, r, s);
  return e == hipSuccess ? ok() : hip_fail(e, "single launch");
}

mx_status moe_mlp_run(const mx_moe_desc& d, const MoeLayout& L, char* w, hipStream_t s) {
  if (d.flags & MX_SINGLE_LAUNCH) return moe_mlp_single(d, L, w, s);
  hipError_t e;
  int32_t* status = reinterpret_cast<int32_t*>(w + L.status);
  const int32_t* idx;
  const float* tw;
  // small batches: the router launch computes the logits (or their partial sums over H) only and
  // the permutation launch makes the top-k selection first (one launch fewer)
  bool select_in_permute = false;
  // decode-sized batches on the spread router: selection and permutation as one launch, which
  // counts its workgroups in on status[2] (set to zero by the router launch)
  bool select_permute = false;
  float* sel_logits = nullptr;
  float* rpart = nullptr;
  int n_part = 0;
  if (d.topk_idx_in == nullptr) {
    float* logits = d.logits_out ? d.logits_out : reinterpret_cast<float*>(w + L.logits);
    int32_t* oi = d.topk_idx_out ? d.topk_idx_out : reinterpret_cast<int32_t*>(w + L.idx);
    float* ow = d.topk_w_out ? d.topk_w_out : reinterpret_cast<float*>(w + L.w);
    select_in_permute = mx::route_logits_defers_select(d.T, d.E, d.k);
    select_permute = L.pcounts_bytes == 0 && mx::route_select_permute_fits(d.T, d.H, d.E, d.k);
    // the router's partial sums borrow the down projection's output rows (written later)
    const size_t part_bytes = (size_t)mx::route_partial_splits(d.T, d.H, d.E) * d.T * d.E * 4;
    rpart = part_bytes <= (size_t)d.T * d.k * d.H * 4 ? reinterpret_cast<float*>(w + L.y) : nullptr;
    {
      ProfScope ps(PK_ROUTE, s);
      e = (select_in_permute || select_permute)
              ? mx::launch_route_logits(d.x, d.wr, d.br, d.T, d.H, d.E, logits, rpart, &n_part, s,
                                        select_permute ? status + 2 : nullptr)
              : mx::launch_route_topk(d.x, d.wr, d.br, d.T, d.H, d.E, d.k, logits, oi, ow, rpart, s);
    }
    if (e != hipSuccess) return hip_fail(e, "route launch");
    sel_logits = logits;
    idx = oi;
    tw = ow;
  } else {
    idx = d.topk_idx_in;
    tw = d.topk_w_in;
  }
  int32_t* offsets = reinterpret_cast<int32_t*>(w + L.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(w + L.perm);
  int32_t* inv = reinterpret_cast<int32_t*>(w + L.inv);
  int2* tiles = reinterpret_cast<int2*>(w + L.tiles);
  {
    ProfScope ps(PK_PERMUTE, s);
    e = select_permute
            ? mx::launch_route_select_permute(sel_logits, rpart, n_part, d.br, d.T, d.E, d.k,
                                              const_cast<int32_t*>(idx), const_cast<float*>(tw),
                                              status + 2, offsets, perm, inv, status, L.tile_rows,
                                              tiles, status + 1, s)
        : select_in_permute
            ? mx::launch_select_permute(sel_logits, rpart, n_part, d.br, d.T, d.k, d.E,
                                        const_cast<int32_t*>(idx), const_cast<float*>(tw), offsets,
                                        perm, inv, status, L.tile_rows, tiles, status + 1, s)
        : L.pcounts_bytes > 0
            ? mx::launch_permute_sliced(idx, d.T, d.k, d.E, offsets, perm, inv, status, L.tile_rows,
                                        tiles, status + 1, reinterpret_cast<int32_t*>(w + L.pcounts), s)
            : mx::launch_permute(idx, d.T, d.k, d.E, offsets, perm, inv, status, L.tile_rows, tiles,
                                 status + 1, s);
  }
  if (e != hipSuccess) return hip_fail(e, "permute launch");
  const bool mx_act = (d.flags & MX_ACT_MXFP4) != 0;
  if (mx_act) {
    // activation variant: x quantized along H in 32-blocks (the same rule as the weights), its
    // scales block-major in pair order; prefill-shaped calls then copy the codes into pair
    // order, tiled (the layouts the gate_up stages read)
    ProfScope ps(PK_QUANTIZE, s);
    const int64_t pitch = ((int64_t)d.T * d.k + 3) / 4 * 4;
    uint8_t* xq = reinterpret_cast<uint8_t*>(w + L.xq);
    uint8_t* xqs = reinterpret_cast<uint8_t*>(w + L.xqs);
    if (L.tile_rows != 16) {
      uint8_t* xq_tok = reinterpret_cast<uint8_t*>(w + L.xq_tok);
      uint8_t* xs_tok = reinterpret_cast<uint8_t*>(w + L.xqs_tok);
      e = mx::launch_quantize(d.x, true, (int64_t)d.T * (d.H / 32), xq_tok, xs_tok, s);
      if (e == hipSuccess)
        e = mx::launch_x_pair_copy(xq_tok, xs_tok, d.H, perm, d.k, d.T * d.k, pitch, xq, xqs, s);
    } else {
      e = mx::launch_quantize_x_scatter(d.x, d.T, d.H, inv, d.k, pitch, xq, xqs, s);
    }
    if (e != hipSuccess) return hip_fail(e, "x quantize launch");
  }
  const mx::MoeGemmArgs g = gemm_args(d, L, w, idx, tw);
  {
    ProfScope ps(PK_GATE_UP, s);
    e = mx::launch_moe_gate_up(g, s);
  }
  if (e != hipSuccess) return hip_fail(e, "gate_up launch");
  {
    ProfScope ps(PK_DOWN, s);
    e = mx::launch_moe_down(g, s);
  }
  if (e != hipSuccess) return hip_fail(e, "down launch");
  {
    ProfScope ps(PK_COMBINE, s);
    e = mx::launch_moe_combine(g, s);
  }
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}
}  // namespace

// Linear workspace: [quantized x, its scales] (MX_ACT_MXFP4) then [fp32 partial sums of the K
// splits] (decode-sized M).
static size_t linear_xq_bytes(int32_t M, int32_t K, uint32_t flags) {
  return (flags & MX_ACT_MXFP4) ? align256((size_t)M * K / 2) + align256((size_t)M * K / 32) : 0;
}
static size_t linear_part_bytes(int32_t M, int32_t K, int32_t N) {
  if (M <= 0 || K < 32 || N <= 0) return 0;
  const int S = mx::linear_k_splits(M, K, N);
  return S > 1 ? align256((size_t)S * M * N * 4) : 0;
}

MX_API size_t mxfp4_linear_workspace(int32_t M, int32_t K, int32_t N, uint32_t flags) {
  if (M < 0 || K < 0 || N < 0) return 0;
  return linear_xq_bytes(M, K, flags) + linear_part_bytes(M, K, N);
}

MX_API mx_status mxfp4_linear(const uint16_t* x, int32_t M, int32_t K, const uint8_t* packed,
                              const uint8_t* scales, int32_t N, void* y, mx_dtype y_dtype,
                              uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  if (y_dtype != MX_F32 && y_dtype != MX_BF16) return fail(MX_ERR_DTYPE, "y_dtype %d", (int)y_dtype);
  if (M < 0 || N < 0 || K <= 0 || K % 32 || K > MX_MAX_K) return fail(MX_ERR_SHAPE, "M=%d K=%d N=%d (K a multiple of 32, <= %d)", M, K, N, MX_MAX_K);
  if (flags & ~MX_ACT_MXFP4) return fail(MX_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  if ((int64_t)M * K * 2 >= (1LL << 31) || (int64_t)N * (K / 2) >= (1LL << 31))
    return fail(MX_ERR_SHAPE, "x and the packed weight must each stay below 2 GiB");
  if (M == 0 || N == 0) return ok();
  if (!x || !packed || !scales || !y) return fail(MX_ERR_NULL, "x, packed, scales and y are required");
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 16) || !aligned(y, 16)) return fail(MX_ERR_ALIGN, "x, packed, scales and y must be 16-byte aligned");
  const size_t need = mxfp4_linear_workspace(M, K, N, flags);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return fail(MX_ERR_WORKSPACE, "workspace too small (%zu bytes needed)", need);
    if (!aligned(ws, 256)) return fail(MX_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  mx_status st = check_device();
  if (st != MX_OK) return st;
  float* partials = linear_part_bytes(M, K, N) > 0
                        ? reinterpret_cast<float*>(static_cast<char*>(ws) + linear_xq_bytes(M, K, flags))
                        : nullptr;
  if (flags & MX_ACT_MXFP4) {
    uint8_t* xq = static_cast<uint8_t*>(ws);
    uint8_t* xqs = xq + align256((size_t)M * K / 2);
    hipError_t e;
    {
      ProfScope ps(PK_QUANTIZE, (hipStream_t)stream);
      e = mx::launch_quantize(x, true, (int64_t)M * (K / 32), xq, xqs, (hipStream_t)stream);
    }
    if (e != hipSuccess) return hip_fail(e, "x quantize launch");
    ProfScope ps(PK_LINEAR, (hipStream_t)stream);
    e = mx::launch_linear_mxact(xq, xqs, M, K, packed, scales, N, y, y_dtype == MX_BF16, partials,
                                (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "linear launch");
  }
  ProfScope ps(PK_LINEAR, (hipStream_t)stream);
  hipError_t e = mx::launch_linear(x, M, K, packed, scales, N, y, y_dtype == MX_BF16, partials,
                                   (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "linear launch");
}

MX_API const char* mx_last_error(void) { return g_err; }

MX_API mx_status mx_get_device_error(void* stream, int32_t* code_host) {
  if (!code_host) return fail(MX_ERR_NULL, "code_host is required");
  mx_status st = check_device();
  if (st != MX_OK) return st;
  int32_t* word = mx::device_error_word();
  if (word == nullptr) return fail(MX_ERR_HIP, "device error word lookup failed");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess) e = hipMemcpy(code_host, word, sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(word, 0, sizeof(int32_t));
  return e == hipSuccess ? ok() : hip_fail(e, "device error read");
}

MX_API mx_status mx_workspace_status(const void* ws, void* stream, int32_t* status) {
  if (!ws || !status) return fail(MX_ERR_NULL, "ws and status are required");
  hipError_t e = hipMemcpyAsync(status, ws, sizeof(int32_t), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "status read");
}

MX_API mx_status mx_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (const ProfRec& r : g_prof_recs) {
    hipEventSynchronize(r.b);
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  g_prof_on.store(enable != 0);
  return ok();
}

MX_API int32_t mx_profile_read(mx_kernel_time* out, int32_t max) {
  double total[PK_COUNT] = {0};
  int32_t count[PK_COUNT] = {0};
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (const ProfRec& r : g_prof_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      total[r.kind] += ms;
      count[r.kind] += 1;
    }
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  int32_t n = 0;
  for (int k = 0; k < PK_COUNT; ++k) {
    if (count[k] == 0) continue;
    if (out && n < max) out[n] = mx_kernel_time{kProfNames[k], count[k], total[k]};
    ++n;
  }
  return n;
}

MX_API const char* mx_version(void) { return "mxfp4moe 0.1 (gfx950)"; }
