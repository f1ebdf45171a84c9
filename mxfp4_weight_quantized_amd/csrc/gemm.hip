// gemm.hip -- MXFP4 weight-only matrix products on gfx950: the MoE MLP's gate_up (fused SwiGLU)
// and down (routing-weight scaled, un-permuted store) grouped GEMMs, the dense linear, and the
// combine over the k experts of each token.
//
// The packed weights are never expanded in memory: they stream from HBM into LDS as 16-byte
// chunks (direct global->LDS loads, several stages in flight) and are decoded in registers right
// before the bf16 MFMA (v_cvt_scalef32_pk_bf16_fp4: two E2M1 codes times the block's E8M0 scale
// per instruction). That is the design the pages point at: quantized matmuls that read the packed
// weights without expanding them ("Hugging Face Transformers GGUF 지원", section "ggml Metal 커널
// 통합") and dedicated MXFP4 kernels instead of a bf16 fallback ("Transformers 4.40 performance
// upgrades for OpenAI GPT-OSS ...", section "MXFP4 4-Bit Quantization").
//
// Operand mapping (v_mfma_f32_16x16x32_bf16). The reduction order inside a product does not
// matter, so the K axis is assigned to lanes in whole 32-element blocks: in one "super-step" of
// four MFMAs, lane group g = lane/16 owns block 4j+g of the K tile, and MFMA s uses elements
// [8s, 8s+8) of it. A lane therefore reads one whole 16-byte packed block (one scale byte) per
// super-step and 64 contiguous bytes of the bf16 activation row.
//
// LDS layout per stage: A [BM rows][KT*64 B], B [BN rows][KT*16 B], 16-byte chunks XOR-swizzled
// by row so that the per-lane 16-byte reads of 8 consecutive rows hit distinct bank groups. The
// swizzle is applied on the load side by choosing which global chunk each lane fetches (the LDS
// destination of a direct load is fixed: lane i writes base + 16*i).
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {
namespace {

enum { MODE_LINEAR = 0, MODE_GATE_UP = 1, MODE_DOWN = 2 };

struct GemmKArgs {
  const uint16_t* A;          // bf16 activation rows of length K
  const int32_t* a_gather;    // A row of permuted row r = a_gather[r] / a_div (NULL: r)
  int a_div;
  const uint8_t* Bp;          // packed weights, expert-major
  const uint8_t* Bs;          // scales, expert-major
  int64_t b_rows_per_expert;  // weight rows per expert (2F gate_up, H down, N linear)
  int64_t bs_total;           // bytes in the whole scale array (bounds the scale copy)
  int N;                      // output columns (F for gate_up)
  int K;
  const int2* tiles;          // grouped: (expert, first permuted row); NULL = dense
  const int32_t* num_tiles;
  const int32_t* offsets;     // grouped: expert row offsets [E+1]
  int M;                      // dense rows
  int F;                      // gate_up: up rows start at F
  void* out;
  int out_bf16;
  const int32_t* perm;        // down: output row index perm[r]
  const float* rw;            // down: routing weight of each pair
};

template <int KT>
__device__ __forceinline__ int swz_b(int row) {
  static_assert(KT == 4 || KT == 8 || KT == 16, "K tile");
  constexpr int SH = KT == 4 ? 2 : (KT == 8 ? 1 : 0);
  return (row >> SH) & (KT - 1);
}

template <int LPS, int STAGES>
__device__ __forceinline__ void wait_stage(int ahead) {
  // ahead = number of later stages already issued (0 .. STAGES-2)
  if constexpr (STAGES >= 4) {
    if (ahead >= 2) { wait_vmcnt<2 * LPS>(); return; }
  }
  if constexpr (STAGES >= 3) {
    if (ahead >= 1) { wait_vmcnt<LPS>(); return; }
  }
  wait_vmcnt<0>();
}

template <int BM, int BN, int WM, int WN, int KT, int STAGES, int MODE, int NBMAX>
__device__ __forceinline__ void gemm_body(const GemmKArgs& p) {
  constexpr int NW = WM * WN;
  constexpr int NT = NW * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr bool SWIGLU = (MODE == MODE_GATE_UP);
  constexpr int BNH = BN / 2;
  constexpr int A_ROW = KT * 64, B_ROW = KT * 16;
  constexpr int A_STAGE = BM * A_ROW, B_STAGE = BN * B_ROW;
  constexpr int IA = A_STAGE / 1024 / NW;
  constexpr int IB = B_STAGE / 1024 / NW;
  constexpr int LPS = IA + IB;
  static_assert(IA * NW * 1024 == A_STAGE && IB * NW * 1024 == B_STAGE, "stage split");
  static_assert(FM * 16 * WM == BM && FN * 16 * WN == BN, "wave tile");
  static_assert(!SWIGLU || FN % 2 == 0, "gate/up fragment pairs");
  static_assert(KT % 4 == 0 && STAGES >= 2 && STAGES <= 4, "pipeline");
  static_assert((STAGES - 1) * LPS < 64, "vmcnt range");
  constexpr int SC_ROWS = SWIGLU ? BNH : BN;
  constexpr int SC_REGION = (SC_ROWS * NBMAX + 16 + 15) / 16 * 16;
  constexpr int SC_BYTES = SWIGLU ? 2 * SC_REGION : SC_REGION;

  __shared__ __attribute__((aligned(1024))) uint8_t sA[STAGES][A_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB[STAGES][B_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sS[SC_BYTES];
  __shared__ int sArow[BM];
  __shared__ int sMis[2];

  // ---- which tile ----
  int e, r0, row_end;
  if (p.tiles != nullptr) {
    if ((int)blockIdx.x >= *p.num_tiles) return;
    const int2 t = p.tiles[blockIdx.x];
    e = t.x;
    r0 = t.y;
    row_end = p.offsets[e + 1];
  } else {
    e = 0;
    r0 = blockIdx.x * BM;
    row_end = p.M;
  }
  const int nt = blockIdx.y;
  const int K = p.K;
  const int nb = K >> 5;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int ln = lane & 15, g = lane >> 4;

  // ---- activation row table, scale copy ----
  for (int i = tid; i < BM; i += NT) {
    const int r = min(r0 + i, row_end - 1);
    sArow[i] = p.a_gather ? p.a_gather[r] / p.a_div : r;
  }
#pragma unroll
  for (int rg = 0; rg < (SWIGLU ? 2 : 1); ++rg) {
    const int64_t first_row = (int64_t)e * p.b_rows_per_expert +
                              (SWIGLU ? (rg ? (int64_t)p.F + nt * BNH : (int64_t)nt * BNH)
                                      : (int64_t)nt * BN);
    const int64_t gstart = first_row * nb;
    const int64_t gend = min(gstart + (int64_t)SC_ROWS * nb, p.bs_total);
    const int64_t abase = gstart & ~(int64_t)3;
    if (tid == 0) sMis[rg] = (int)(gstart - abase);
    const int ndw = (int)((gend - abase + 3) >> 2);
    for (int i = tid; i < ndw; i += NT) {
      const int64_t off = abase + 4 * (int64_t)i;
      uint32_t v;
      if (off + 4 <= p.bs_total) {
        v = *reinterpret_cast<const uint32_t*>(p.Bs + off);
      } else {
        v = 0;
        for (int b = 0; b < 4; ++b)
          if (off + b < p.bs_total) v |= (uint32_t)p.Bs[off + b] << (8 * b);
      }
      *reinterpret_cast<uint32_t*>(sS + rg * SC_REGION + 4 * i) = v;
    }
  }
  __syncthreads();

  // ---- per-lane global sources of the direct-to-LDS loads ----
  const uint16_t* aptr[IA];
  int achunk[IA];
#pragma unroll
  for (int q = 0; q < IA; ++q) {
    const int off = (wave * IA + q) * 1024 + lane * 16;
    const int lrow = off / A_ROW;
    const int chunk = ((off % A_ROW) >> 4) ^ (lrow & 7);
    achunk[q] = chunk;
    aptr[q] = p.A + (int64_t)sArow[lrow] * K + chunk * 8;
  }
  const uint8_t* bptr[IB];
  int bchunk[IB];
#pragma unroll
  for (int q = 0; q < IB; ++q) {
    const int off = (wave * IB + q) * 1024 + lane * 16;
    const int lrow = off / B_ROW;
    const int chunk = ((off % B_ROW) >> 4) ^ swz_b<KT>(lrow);
    int grow;
    if (SWIGLU)
      grow = lrow < BNH ? min(nt * BNH + lrow, p.F - 1) : p.F + min(nt * BNH + lrow - BNH, p.F - 1);
    else
      grow = min(nt * BN + lrow, p.N - 1);
    bchunk[q] = chunk;
    bptr[q] = p.Bp + ((int64_t)e * p.b_rows_per_expert + grow) * (K >> 1) + chunk * 16;
  }

  auto issue = [&](int kt, int st) {
#pragma unroll
    for (int q = 0; q < IA; ++q) {
      const int blk = kt * KT + (achunk[q] >> 2);
      const uint16_t* src = blk < nb ? aptr[q] + kt * KT * 32 : aptr[q] - achunk[q] * 8;
      load_lds_16(src, &sA[st][(wave * IA + q) * 1024]);
    }
#pragma unroll
    for (int q = 0; q < IB; ++q) {
      const int blk = kt * KT + bchunk[q];
      const uint8_t* src = blk < nb ? bptr[q] + kt * KT * 16 : bptr[q] - bchunk[q] * 16;
      load_lds_16(src, &sB[st][(wave * IB + q) * 1024]);
    }
  };

  // ---- per-lane LDS read coordinates ----
  int brow[FN], scoff[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    int base;
    if (SWIGLU)
      base = (f < FN / 2) ? wn * (BNH / WN) + f * 16 : BNH + wn * (BNH / WN) + (f - FN / 2) * 16;
    else
      base = wn * TN + f * 16;
    brow[f] = base + ln;
    const int rg = SWIGLU ? (brow[f] >= BNH) : 0;
    scoff[f] = rg * SC_REGION + sMis[rg] + (brow[f] - rg * BNH) * nb;
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntk = (nb + KT - 1) / KT;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < ntk) issue(s, s);

  for (int kt = 0; kt < ntk; ++kt) {
    wait_stage<LPS, STAGES>(min(ntk - 1 - kt, STAGES - 2));
    barrier_lds();
    if (kt + STAGES - 1 < ntk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    const int st = kt % STAGES;
    const uint8_t* As = sA[st];
    const uint8_t* Bs = sB[st];
    const bool tail = (kt + 1) * KT > nb;
#pragma unroll
    for (int j = 0; j < KT / 4; ++j) {
      const int blk = kt * KT + 4 * j + g;
      const bool kval = !tail || blk < nb;
      bf16x8 bf[FN][4];
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const int r = brow[f];
        const u32x4 w = lds_read_b128(Bs + r * B_ROW + (((4 * j + g) ^ swz_b<KT>(r)) << 4));
        const float sc = e8m0_to_f32(sS[scoff[f] + (kval ? blk : 0)]);
#pragma unroll
        for (int s = 0; s < 4; ++s) bf[f][s] = fp4x8_to_bf16x8(kval ? w[s] : 0u, sc);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * TM + i * 16 + ln;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          u32x4 a = lds_read_b128(As + r * A_ROW + ((((4 * j + g) * 4 + s) ^ (r & 7)) << 4));
          if (!kval) a = u32x4{0u, 0u, 0u, 0u};
          const bf16x8 av = u32x4_as_bf16x8(a);
#pragma unroll
          for (int f = 0; f < FN; ++f) acc[i][f] = mfma16x16x32(av, bf[f][s], acc[i][f]);
        }
      }
    }
  }

  // ---- epilogue ----
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = r0 + wm * TM + i * 16 + 4 * g + q;
      if (r >= row_end) continue;
      if constexpr (MODE == MODE_GATE_UP) {
        uint16_t* h = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
        for (int f = 0; f < FN / 2; ++f) {
          const int col = nt * BNH + wn * (BNH / WN) + f * 16 + ln;
          if (col >= p.F) continue;
          const float gt = acc[i][f][q], up = acc[i][FN / 2 + f][q];
          const float hv = gt / (1.f + expf(-gt)) * up;
          h[(int64_t)r * p.F + col] = (uint16_t)f32_to_bf16_bits(hv);
        }
      } else if constexpr (MODE == MODE_DOWN) {
        const int pair = p.perm[r];
        const float wgt = p.rw[pair];
        float* y = reinterpret_cast<float*>(p.out);
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int col = nt * BN + wn * TN + f * 16 + ln;
          if (col < p.N) y[(int64_t)pair * p.N + col] = acc[i][f][q] * wgt;
        }
      } else {
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int col = nt * BN + wn * TN + f * 16 + ln;
          if (col >= p.N) continue;
          if (p.out_bf16)
            reinterpret_cast<uint16_t*>(p.out)[(int64_t)r * p.N + col] =
                (uint16_t)f32_to_bf16_bits(acc[i][f][q]);
          else
            reinterpret_cast<float*>(p.out)[(int64_t)r * p.N + col] = acc[i][f][q];
        }
      }
    }
  }
}

// One kernel name per role, so profiles show which product a launch is.
template <int BM, int BN, int WM, int WN, int KT, int ST, int NBM>
__global__ __launch_bounds__(WM * WN * 64) void moe_gate_up_swiglu_kernel(GemmKArgs p) {
  gemm_body<BM, BN, WM, WN, KT, ST, MODE_GATE_UP, NBM>(p);
}
template <int BM, int BN, int WM, int WN, int KT, int ST, int NBM>
__global__ __launch_bounds__(WM * WN * 64) void moe_down_weighted_kernel(GemmKArgs p) {
  gemm_body<BM, BN, WM, WN, KT, ST, MODE_DOWN, NBM>(p);
}
template <int BM, int BN, int WM, int WN, int KT, int ST, int NBM>
__global__ __launch_bounds__(WM * WN * 64) void linear_kernel(GemmKArgs p) {
  gemm_body<BM, BN, WM, WN, KT, ST, MODE_LINEAR, NBM>(p);
}

// out[t][n] = sum_{j < k} Y[t*k + j][n] in slot order; pairs with inv < 0 (skipped routing
// indices) contribute nothing.
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Y,
                                                      const int32_t* __restrict__ inv, int T,
                                                      int H, int k, void* __restrict__ out) {
  const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int h4 = H >> 2;
  if (i4 >= (int64_t)T * h4) return;
  const int t = (int)(i4 / h4);
  const int c = (int)(i4 % h4) * 4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    if (inv[(int64_t)t * k + j] < 0) continue;
    const float4 v = *reinterpret_cast<const float4*>(Y + ((int64_t)t * k + j) * H + c);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  if (BF16_OUT) {
    const uint32_t lo = f32_to_bf16_bits(s.x) | (f32_to_bf16_bits(s.y) << 16);
    const uint32_t hi = f32_to_bf16_bits(s.z) | (f32_to_bf16_bits(s.w) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (int64_t)t * H + c) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (int64_t)t * H + c) = s;
  }
}

// ---- tile configurations ----
// Decode-shaped (few rows per expert): 16-row tiles, weight streaming dominates.
// Prefill-shaped: 128 x 128 tiles, MFMA dominates.
constexpr int kNBMax = 96;          // scale blocks per row held in LDS (K <= 3072)
constexpr int kNBMaxLarge = 256;    // K <= 8192 (decode tiles only)

template <int BM, int BN, int WM, int WN, int KT, int ST, int MODE, int NBM>
hipError_t launch_gemm(const GemmKArgs& a, int grid_x, int n_cols_tiles, hipStream_t stream) {
  if (grid_x <= 0 || n_cols_tiles <= 0) return hipSuccess;
  const dim3 grid(grid_x, n_cols_tiles), block(WM * WN * 64);
  if constexpr (MODE == MODE_GATE_UP)
    hipLaunchKernelGGL((moe_gate_up_swiglu_kernel<BM, BN, WM, WN, KT, ST, NBM>), grid, block, 0, stream, a);
  else if constexpr (MODE == MODE_DOWN)
    hipLaunchKernelGGL((moe_down_weighted_kernel<BM, BN, WM, WN, KT, ST, NBM>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((linear_kernel<BM, BN, WM, WN, KT, ST, NBM>), grid, block, 0, stream, a);
  return hipGetLastError();
}

bool use_prefill_tiles(int T, int k, int E) { return (int64_t)T * k >= 48LL * E; }

}  // namespace

int moe_tile_rows(int T, int k, int E) { return use_prefill_tiles(T, k, E) ? 128 : 16; }

int moe_max_tiles(int T, int k, int E, int tile_rows) {
  return (int)(((int64_t)T * k + tile_rows - 1) / tile_rows) + E;
}

hipError_t launch_moe_gate_up(const MoeGemmArgs& m, hipStream_t stream) {
  // A = x rows gathered through perm / k, B = W_gu[e] (2F rows), out = h [P][F]
  GemmKArgs g{};
  g.A = m.x;
  g.a_gather = m.perm;
  g.a_div = m.k;
  g.Bp = m.gu_packed;
  g.Bs = m.gu_scales;
  g.b_rows_per_expert = 2LL * m.F;
  g.bs_total = (int64_t)m.E * 2 * m.F * (m.H / 32);
  g.N = m.F;
  g.K = m.H;
  g.tiles = m.tiles;
  g.num_tiles = m.num_tiles;
  g.offsets = m.offsets;
  g.F = m.F;
  g.out = m.h;
  if (use_prefill_tiles(m.T, m.k, m.E))
    return launch_gemm<128, 128, 2, 2, 4, 3, MODE_GATE_UP, kNBMax>(g, m.max_tiles, (m.F + 63) / 64, stream);
  return launch_gemm<16, 64, 1, 2, 8, 4, MODE_GATE_UP, kNBMax>(g, m.max_tiles, (m.F + 31) / 32, stream);
}

hipError_t launch_moe_down(const MoeGemmArgs& m, hipStream_t stream) {
  // A = h rows (permuted order), B = W_dn[e] (H rows), out = Y[pair] * routing weight
  GemmKArgs d{};
  d.A = m.h;
  d.a_gather = nullptr;
  d.a_div = 1;
  d.Bp = m.dn_packed;
  d.Bs = m.dn_scales;
  d.b_rows_per_expert = m.H;
  d.bs_total = (int64_t)m.E * m.H * (m.F / 32);
  d.N = m.H;
  d.K = m.F;
  d.tiles = m.tiles;
  d.num_tiles = m.num_tiles;
  d.offsets = m.offsets;
  d.F = m.F;
  d.out = m.y;
  d.perm = m.perm;
  d.rw = m.topk_w;
  if (use_prefill_tiles(m.T, m.k, m.E))
    return launch_gemm<128, 128, 2, 2, 4, 3, MODE_DOWN, kNBMax>(d, m.max_tiles, (m.H + 127) / 128, stream);
  return launch_gemm<16, 64, 1, 4, 8, 4, MODE_DOWN, kNBMax>(d, m.max_tiles, (m.H + 63) / 64, stream);
}

hipError_t launch_moe_combine(const MoeGemmArgs& m, hipStream_t stream) {
  const int64_t n4 = (int64_t)m.T * (m.H / 4);
  const unsigned grid = (unsigned)((n4 + 255) / 256);
  if (m.out_bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(grid), dim3(256), 0, stream, m.y, m.inv, m.T, m.H,
                       m.k, m.out);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(grid), dim3(256), 0, stream, m.y, m.inv, m.T,
                       m.H, m.k, m.out);
  return hipGetLastError();
}

hipError_t launch_linear(const uint16_t* x, int M, int K, const uint8_t* packed,
                         const uint8_t* scales, int N, void* y, bool y_bf16, hipStream_t stream) {
  GemmKArgs g{};
  g.A = x;
  g.a_div = 1;
  g.Bp = packed;
  g.Bs = scales;
  g.b_rows_per_expert = N;
  g.bs_total = (int64_t)N * (K / 32);
  g.N = N;
  g.K = K;
  g.M = M;
  g.F = N;
  g.out = y;
  g.out_bf16 = y_bf16 ? 1 : 0;
  const int nb = K / 32;
  if (M > 64 && nb <= kNBMax)
    return launch_gemm<128, 128, 2, 2, 4, 3, MODE_LINEAR, kNBMax>(g, (M + 127) / 128, (N + 127) / 128, stream);
  if (nb <= kNBMax)
    return launch_gemm<16, 64, 1, 4, 8, 4, MODE_LINEAR, kNBMax>(g, (M + 15) / 16, (N + 63) / 64, stream);
  return launch_gemm<16, 64, 1, 4, 8, 3, MODE_LINEAR, kNBMaxLarge>(g, (M + 15) / 16, (N + 63) / 64, stream);
}

hipError_t gemm_init() { return hipSuccess; }

}  // namespace mx
