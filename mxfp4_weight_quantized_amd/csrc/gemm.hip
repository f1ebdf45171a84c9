// gemm.hip -- launches of the MoE MLP's gate_up (fused SwiGLU) and down grouped GEMMs, the dense
// linear and the combine over the k experts of each token, one kernel per product; the tile
// itself is gemm_tile.h.
#include "gemm_tile.h"

namespace mx {
namespace {

// ---- which tile ----
// Workgroups go round-robin to the 8 XCDs (each with its own L2). XCD x takes super-tiles x, x+8,
// ...; a super-tile is GM x GN (m, n) tiles, and its GM*GN workgroups run together on the XCD, so
// at every K stage they share GM activation tiles and GN weight tiles in L2. Returns false for a
// workgroup past the last tile. Grouped tiles come from the tile list: (expert, first row).
template <int BM, int GM>
__device__ __forceinline__ bool pick_tile(const GemmKArgs& p, int& e, int& r0, int& row_end,
                                          int& nt) {
  const int GN = p.gn;
  const bool grouped = p.tiles != nullptr;
  const int num_mt = grouped ? *p.num_tiles : (p.M + BM - 1) / BM;
  const int sm_count = (num_mt + GM - 1) / GM, sn_count = (p.n_tiles + GN - 1) / GN;
  const int slot = blockIdx.x >> 3;
  const int super_tile = (blockIdx.x & 7) + 8 * (slot / (GM * GN));
  if (super_tile >= sm_count * sn_count) return false;
  const int pos = slot % (GM * GN);
  const int mt = (super_tile % sm_count) * GM + pos / GN;
  nt = (super_tile / sm_count) * GN + pos % GN;
  if (mt >= num_mt || nt >= p.n_tiles) return false;
  if (grouped) {
    const int2 tl = p.tiles[mt];
    e = __builtin_amdgcn_readfirstlane(tl.x);
    r0 = __builtin_amdgcn_readfirstlane(tl.y);
    row_end = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);
  } else {
    e = 0;
    r0 = mt * BM;
    row_end = p.M;
  }
  return true;
}

template <int BM, int BN, int WM, int WN, int KT, int STAGES, int MODE, int GM, bool AFP4, int SCM,
          bool TW, int MF>
__device__ __forceinline__ void gemm_body(const GemmKArgs& p) {
  __shared__ typename GemmLds<BM, BN, WM, WN, KT, STAGES, MODE, AFP4, SCM, TW>::Storage sm;
  int e, r0, row_end, nt;
  if (!pick_tile<BM, GM>(p, e, r0, row_end, nt)) return;
  gemm_tile<BM, BN, WM, WN, KT, STAGES, MODE, AFP4, SCM, TW, MF, GM == 1 && MODE != MODE_LINEAR>(
      p, sm, e, r0, row_end, nt);
}

// One kernel name per role, so profiles show which product a launch is.
template <int BM, int BN, int WM, int WN, int KT, int ST, int GM, int OCC, bool AFP4, int SCM, bool TW, int MF>
__global__ __launch_bounds__(WM * WN * 64, (OCC * WM * WN + 3) / 4) void moe_gate_up_swiglu_kernel(GemmKArgs p) {
  gemm_body<BM, BN, WM, WN, KT, ST, MODE_GATE_UP, GM, AFP4, SCM, TW, MF>(p);
}
template <int BM, int BN, int WM, int WN, int KT, int ST, int GM, int OCC, bool AFP4, int SCM, bool TW, int MF>
__global__ __launch_bounds__(WM * WN * 64, (OCC * WM * WN + 3) / 4) void moe_down_weighted_kernel(GemmKArgs p) {
  gemm_body<BM, BN, WM, WN, KT, ST, MODE_DOWN, GM, AFP4, SCM, TW, MF>(p);
}
template <int BM, int BN, int WM, int WN, int KT, int ST, int GM, int OCC, bool AFP4, int SCM, int MF>
__global__ __launch_bounds__(WM * WN * 64, (OCC * WM * WN + 3) / 4) void linear_kernel(GemmKArgs p) {
  gemm_body<BM, BN, WM, WN, KT, ST, MODE_LINEAR, GM, AFP4, SCM, false, MF>(p);
}
// The combine with one workgroup per token (the per-step path): the token's KK (row, weight) pairs
// are the same for the whole workgroup, so they come through the scalar cache and the vector
// memory path carries only the rows. Each thread takes 8 columns and issues the loads of all KK
// rows before summing. The arithmetic is combine8's (each product w * Y, or w * (Y + bias),
// rounded to fp32, then added in slot order), so both give the same bits: a pair whose row index
// lies outside [0, P) (a skipped routing index) reads row 0 and adds +0 instead of its product,
// which leaves the sum unchanged (it starts at +0 and cannot become -0).
constexpr int kCombineThreads = 384;  // 8 columns per thread: H <= 3072
constexpr int kMaxTopK = 8;           // experts per token (the C ABI's limit)
template <bool BF16_OUT, int KK>
__global__ __launch_bounds__(kCombineThreads) void combine_token_kernel(
    const float* __restrict__ Y, const int32_t* __restrict__ inv, const float* __restrict__ w,
    int H, int P, void* __restrict__ out, const int32_t* __restrict__ idx,
    const float* __restrict__ bias) {
#pragma clang fp contract(off)  // each product rounded before it is added (no fused multiply-add)
  const int64_t t = blockIdx.x;
  const int c = threadIdx.x * 8;
  if (c >= H) return;
  int r[KK];
  bool ok[KK];
  float wj[KK];
#pragma unroll
  for (int j = 0; j < KK; ++j) {
    const int rr = inv[t * KK + j];
    ok[j] = rr >= 0 && rr < P;
    r[j] = ok[j] ? rr : 0;
    wj[j] = w[t * KK + j];
  }
  f32x4 v0[KK], v1[KK];
#pragma unroll
  for (int j = 0; j < KK; ++j) {
    v0[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Y + (int64_t)r[j] * H + c));
    v1[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Y + (int64_t)r[j] * H + c + 4));
  }
  if (bias != nullptr) {
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      const float* bb = bias + (int64_t)(ok[j] ? idx[t * KK + j] : 0) * H + c;
      v0[j] += *reinterpret_cast<const f32x4*>(bb);
      v1[j] += *reinterpret_cast<const f32x4*>(bb + 4);
    }
  }
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KK; ++j) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s[u] += ok[j] ? __fmul_rn(v0[j][u], wj[j]) : 0.f;
      s[4 + u] += ok[j] ? __fmul_rn(v1[j][u], wj[j]) : 0.f;
    }
  }
  if (BF16_OUT) {
    uint32_t q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = f32_to_bf16_bits(s[2 * u]) | (f32_to_bf16_bits(s[2 * u + 1]) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + t * H + c) = make_uint4(q[0], q[1], q[2], q[3]);
  } else {
    float* o = reinterpret_cast<float*>(out) + t * H + c;
    *reinterpret_cast<float4*>(o) = make_float4(s[0], s[1], s[2], s[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(s[4], s[5], s[6], s[7]);
  }
}

template <bool BF16_OUT, int KK>
void launch_combine_k(const MoeGemmArgs& m, const float* bias, hipStream_t stream) {
  const int threads = (m.H / 8 + 63) / 64 * 64;
  hipLaunchKernelGGL((combine_token_kernel<BF16_OUT, KK>), dim3(m.T), dim3(threads), 0, stream,
                     m.y, m.inv, m.topk_w, m.H, m.T * m.k, m.out, m.topk_idx, bias);
}
template <bool BF16_OUT>
void launch_combine(const MoeGemmArgs& m, const float* bias, hipStream_t stream) {
  switch (m.k) {
    case 1: launch_combine_k<BF16_OUT, 1>(m, bias, stream); break;
    case 2: launch_combine_k<BF16_OUT, 2>(m, bias, stream); break;
    case 3: launch_combine_k<BF16_OUT, 3>(m, bias, stream); break;
    case 4: launch_combine_k<BF16_OUT, 4>(m, bias, stream); break;
    case 5: launch_combine_k<BF16_OUT, 5>(m, bias, stream); break;
    case 6: launch_combine_k<BF16_OUT, 6>(m, bias, stream); break;
    case 7: launch_combine_k<BF16_OUT, 7>(m, bias, stream); break;
    default: launch_combine_k<BF16_OUT, kMaxTopK>(m, bias, stream); break;
  }
}

// Split linear: out[i] = sum over z of part[z * n + i], in split order, as fp32 or bf16.
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int S,
                                                           int64_t n, void* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = part[i];
  for (int z = 1; z < S; ++z) s += part[(int64_t)z * n + i];
  if (BF16_OUT) reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_bf16_bits(s);
  else reinterpret_cast<float*>(out)[i] = s;
}


template <class C, int MODE, bool AFP4 = false, int SCM = C::SCM, bool TW = false>
hipError_t launch_gemm(GemmKArgs a, int m_tiles, int n_cols, hipStream_t stream) {
  const int n_tiles = (MODE == MODE_GATE_UP) ? (n_cols + C::BN / 2 - 1) / (C::BN / 2)
                                             : (n_cols + C::BN - 1) / C::BN;
  if (m_tiles <= 0 || n_tiles <= 0) return hipSuccess;
  a.n_tiles = n_tiles;
  // grid: 8 XCDs x (super-tiles per XCD) x (tiles per super-tile), from the row-tile bound.
  // Super-tiles of 32 tiles (activation and weight tiles shared in an XCD's L2; for decode tiles,
  // neighbouring column tiles of one expert, adjacent in memory, streamed by one XCD). Where that
  // gives fewer super-tiles than XCDs (a dense linear of one row tile: 45 column tiles had run
  // on 2 of the 8 XCDs) the groups narrow until every XCD gets one.
  const int m_sup = (m_tiles + C::GM - 1) / C::GM;
  int GN = 32 / C::GM;
  if ((int64_t)m_sup * ((n_tiles + GN - 1) / GN) < 8) GN = std::max(1, n_tiles / ((8 + m_sup - 1) / m_sup));
  a.gn = GN;
  const int64_t supers = (int64_t)m_sup * ((n_tiles + GN - 1) / GN);
  const unsigned zs = (MODE == MODE_LINEAR && a.k_splits > 1) ? (unsigned)a.k_splits : 1u;
  const dim3 grid((unsigned)(8 * C::GM * GN * ((supers + 7) / 8)), 1, zs), block(C::WM * C::WN * 64);
  constexpr int MF = AFP4 ? 16 : C::MF;
  if constexpr (MODE == MODE_GATE_UP)
    hipLaunchKernelGGL((moe_gate_up_swiglu_kernel<C::BM, C::BN, C::WM, C::WN, C::KT, C::ST, C::GM, C::OCC, AFP4, SCM, TW, MF>), grid, block, 0, stream, a);
  else if constexpr (MODE == MODE_DOWN)
    hipLaunchKernelGGL((moe_down_weighted_kernel<C::BM, C::BN, C::WM, C::WN, C::KT, C::ST, C::GM, C::OCC, AFP4, SCM, TW, MF>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((linear_kernel<C::BM, C::BN, C::WM, C::WN, C::KT, C::ST, C::GM, C::OCC, AFP4, SCM, MF>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// Dense linear: prefill tiles above 64 rows, else 16-row tiles. Weight scales are read as whole
// dwords unless the scale array (N * K/32 bytes) is not a whole number of dwords.
template <bool AFP4>
hipError_t launch_linear_tiles(const GemmKArgs& g, int M, int N, hipStream_t stream) {
  const int nb = g.K >> 5;
  const bool dw = ((int64_t)N * nb) % 4 == 0;
  if (M > 64) {
    using C = std::conditional_t<AFP4, CfgPreGU4, CfgPreGU>;
    const int mt = (M + C::BM - 1) / C::BM;
    if constexpr (C::KT % 4 != 0)  // row-major stage scales need 4-block stages
      return launch_gemm<C, MODE_LINEAR, AFP4, SCM_BYTE>(g, mt, N, stream);
    else
      return dw ? launch_gemm<C, MODE_LINEAR, AFP4, SCM_STAGE>(g, mt, N, stream)
                : launch_gemm<C, MODE_LINEAR, AFP4, SCM_BYTE>(g, mt, N, stream);
  }
  const int mt = (M + CfgDecDn128::BM - 1) / CfgDecDn128::BM;
  // (split K: each split needs only its stages' scales)
  if (dw && nb <= kResidentNb && g.k_splits <= 1)
    return launch_gemm<CfgDecDn128, MODE_LINEAR, AFP4, SCM_RESIDENT>(g, mt, N, stream);
  return dw ? launch_gemm<CfgDecDn128, MODE_LINEAR, AFP4, SCM_STAGE>(g, mt, N, stream)
            : launch_gemm<CfgDecDn128, MODE_LINEAR, AFP4, SCM_BYTE>(g, mt, N, stream);
}

bool use_prefill_tiles(int T, int k, int E) { return (int64_t)T * k >= 64LL * E; }

// Split linear: output tiles in fp32 partial sums, then their sum in split order into y.
template <bool AFP4>
hipError_t launch_linear_split(GemmKArgs g, int M, int N, void* y, bool y_bf16, float* partials,
                               hipStream_t stream) {
  const int S = linear_k_splits(M, g.K, N);
  if (S > 1) {
    g.out = partials;
    g.out_bf16 = 0;
    g.k_splits = S;
    g.part_stride = (int64_t)M * N;
  } else {
    g.out = y;
    g.out_bf16 = y_bf16 ? 1 : 0;
  }
  hipError_t e = launch_linear_tiles<AFP4>(g, M, N, stream);
  if (e != hipSuccess || S <= 1) return e;
  const int64_t n = (int64_t)M * N;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (y_bf16)
    hipLaunchKernelGGL(split_reduce_kernel<true>, dim3(grid), dim3(256), 0, stream, partials, S, n, y);
  else
    hipLaunchKernelGGL(split_reduce_kernel<false>, dim3(grid), dim3(256), 0, stream, partials, S, n, y);
  return hipGetLastError();
}

}  // namespace

int moe_tile_rows(int T, int k, int E, bool mx_act) {
  return use_prefill_tiles(T, k, E) ? (mx_act ? kPrefillRows4 : kPrefillRows) : 16;
}

// Each touched expert (at most min(E, T*k) of them) adds at most one partial row tile.
int moe_max_tiles(int T, int k, int E, int tile_rows) {
  return (int)(((int64_t)T * k + tile_rows - 1) / tile_rows + std::min<int64_t>(E, (int64_t)T * k));
}

namespace {
// Row-major weights with stages of other than a multiple of 4 blocks read stage scales bytewise.
template <class C, bool TW>
constexpr int stage_scm() { return (C::SCM == SCM_STAGE && !TW && C::KT % 4 != 0) ? SCM_BYTE : C::SCM; }
template <class C, int MODE, bool AFP4, bool TW>
hipError_t launch_moe_gemm(const GemmKArgs& g, int m_tiles, int n_cols, hipStream_t stream) {
  return launch_gemm<C, MODE, AFP4, stage_scm<C, TW>(), TW>(g, m_tiles, n_cols, stream);
}
template <bool TW>
hipError_t gate_up_tw(GemmKArgs g, const MoeGemmArgs& m, hipStream_t stream) {
  const bool pre = use_prefill_tiles(m.T, m.k, m.E);
  if (m.mx_act) {
    g.A = reinterpret_cast<const uint16_t*>(m.xq);  // packed codes, addressed in bytes
    if (pre) {  // prefill tiles: x's codes already in pair order (tiled), no gather
      g.a_gather = nullptr;
      g.a_rows = (int64_t)m.T * m.k;
    }
    g.Asc = m.xqs;
    g.out = m.hq;  // h leaves the epilogue quantized
    g.out_scales = m.hqs;
    if (pre) return launch_moe_gemm<CfgPreGU4, MODE_GATE_UP, true, TW>(g, m.max_tiles, m.F, stream);
    if (use_tiny_tiles(m.T, m.k, m.E, 2 * m.F))
      return launch_moe_gemm<CfgTinyGU, MODE_GATE_UP, true, TW>(g, m.max_tiles, m.F, stream);
    return launch_moe_gemm<CfgDecGU, MODE_GATE_UP, true, TW>(g, m.max_tiles, m.F, stream);
  }
  if (pre) return launch_moe_gemm<CfgPreGU, MODE_GATE_UP, false, TW>(g, m.max_tiles, m.F, stream);
  if (use_tiny_tiles(m.T, m.k, m.E, 2 * m.F))
    return launch_moe_gemm<CfgTinyGU, MODE_GATE_UP, false, TW>(g, m.max_tiles, m.F, stream);
  return launch_moe_gemm<CfgDecGU, MODE_GATE_UP, false, TW>(g, m.max_tiles, m.F, stream);
}
template <bool TW>
hipError_t down_tw(GemmKArgs d, const MoeGemmArgs& m, hipStream_t stream) {
  const bool pre = use_prefill_tiles(m.T, m.k, m.E);
  if (m.mx_act) {
    d.A = reinterpret_cast<const uint16_t*>(m.hq);
    d.Asc = m.hqs;
    if (pre) return launch_moe_gemm<CfgPreDn4, MODE_DOWN, true, TW>(d, m.max_tiles, m.H, stream);
    if (use_tiny_tiles(m.T, m.k, m.E, m.H))
      return launch_moe_gemm<CfgTinyDn, MODE_DOWN, true, TW>(d, m.max_tiles, m.H, stream);
    return launch_moe_gemm<CfgDecDn, MODE_DOWN, true, TW>(d, m.max_tiles, m.H, stream);
  }
  if (pre) return launch_moe_gemm<CfgPreDn, MODE_DOWN, false, TW>(d, m.max_tiles, m.H, stream);
  if (use_tiny_tiles(m.T, m.k, m.E, m.H))
    return launch_moe_gemm<CfgTinyDn, MODE_DOWN, false, TW>(d, m.max_tiles, m.H, stream);
  return launch_moe_gemm<CfgDecDn, MODE_DOWN, false, TW>(d, m.max_tiles, m.H, stream);
}
}  // namespace

hipError_t launch_moe_gate_up(const MoeGemmArgs& m, hipStream_t stream) {
  const GemmKArgs g = gate_up_args(m);
  return m.tiled ? gate_up_tw<true>(g, m, stream) : gate_up_tw<false>(g, m, stream);
}

hipError_t launch_moe_down(const MoeGemmArgs& m, hipStream_t stream) {
  const GemmKArgs d = down_args(m);
  return m.tiled ? down_tw<true>(d, m, stream) : down_tw<false>(d, m, stream);
}

hipError_t launch_moe_combine(const MoeGemmArgs& m, hipStream_t stream) {
  const float* bias = m.act_custom ? m.dn_bias : nullptr;
  if (m.out_bf16) launch_combine<true>(m, bias, stream);
  else launch_combine<false>(m, bias, stream);
  return hipGetLastError();
}

// Decode-sized dense linears (M <= 64) have few output tiles (45 for N = 5760): each tile's K is
// split over several workgroups, enough for about three per CU while every split keeps at least
// 3 pipeline stages of 4 blocks.
int linear_k_splits(int M, int K, int N) {
  if (M > 64) return 1;
  const int64_t tiles = (int64_t)((M + 15) / 16) * ((N + 127) / 128);
  const int stages = (K / 32 + 3) / 4;
  const int64_t want = (768 + tiles - 1) / tiles;
  return (int)std::max<int64_t>(1, std::min<int64_t>(stages / 3, want));
}

hipError_t launch_linear(const uint16_t* x, int M, int K, const uint8_t* packed,
                         const uint8_t* scales, int N, void* y, bool y_bf16, float* partials,
                         hipStream_t stream) {
  GemmKArgs g{};
  g.A = x;
  g.a_rows = M;
  g.a_div = 1;
  g.Bp = packed;
  g.Bs = scales;
  g.b_rows_per_expert = N;
  g.N = N;
  g.K = K;
  g.M = M;
  g.rows_total = M;
  g.F = N;
  return launch_linear_split<false>(g, M, N, y, y_bf16, partials, stream);
}

hipError_t launch_linear_mxact(const uint8_t* xq, const uint8_t* xqs, int M, int K,
                               const uint8_t* packed, const uint8_t* scales, int N, void* y,
                               bool y_bf16, float* partials, hipStream_t stream) {
  GemmKArgs g{};
  g.A = reinterpret_cast<const uint16_t*>(xq);
  g.Asc = xqs;
  g.a_rows = M;
  g.a_div = 1;
  g.Bp = packed;
  g.Bs = scales;
  g.b_rows_per_expert = N;
  g.N = N;
  g.K = K;
  g.M = M;
  g.rows_total = M;
  g.F = N;
  return launch_linear_split<true>(g, M, N, y, y_bf16, partials, stream);
}

}  // namespace mx
