// route.hip -- router logits, top-k expert selection and softmax over the selected experts.
//
// The GGUF page ("Hugging Face Transformers GGUF 지원", agentlenshq.com, section "ggml Metal 커널
// 통합") names a dedicated top-k kernel for MoE expert selection; the router itself is the
// library's reading: logits = x W_r^T + b, top-k by (logit desc, expert index asc), softmax over
// the k selected logits.
//
// Two kernels. route_logits_kernel: a workgroup takes 16 tokens and G groups of 16 experts; its
// up to 16 waves split H between them (each wave a 16 x 16 logit tile over its share of H, bf16
// MFMA with fp32 accumulate, operands read straight from global memory -- W_r is small and stays
// in L2) and the partial tiles meet in LDS, summed in a fixed order so that the logits do not
// depend on timing. With few tokens G = 1 and the groups spread over many workgroups, so a decode
// batch is not left to a handful of CUs; given a buffer for partial sums, H is then also split
// over 2 or 4 workgroups per tile, whose partial tiles the selection kernel sums in split order.
// With many tokens G covers all experts and each token tile is read once, and the same workgroup
// then ranks its tokens' logits from LDS (no second kernel). Otherwise route_select_kernel: one
// 16-lane row of a wave per token (adds up the partial tiles and the bias first, if there are
// partials) ranks the logits (argmax k times, inside the row) and writes the top-k indices and
// their softmax.
//
// Large batches with a logits buffer take route_tile_kernel instead: 64 tokens per workgroup
// against every expert, operands staged through LDS. The cost of the 16-token kernel above is
// not arithmetic but W_r streaming into every CU again for every 16 tokens (each CU pulls its
// share of L2 at a limited rate); with 64-token tiles that stream is four times shorter, and H is
// split over 2 to 8 workgroups per tile so that the launch still covers the CUs. The splits'
// partial logits go through memory to route_select_kernel, which sums them in split order.
#include "gemm_tile.h"
#include "route_device.h"

namespace mx {
namespace {

constexpr int kTokPerWG = 16;
// Below this many (token tile, expert group) pairs each workgroup takes one expert group, so a
// small batch spreads over more CUs (and selection runs as its own kernel).
constexpr int kSpreadBelow = 512;

// SELECT: the workgroup covers all experts of its tokens (n_groups * 16 >= E); it keeps the
// logits tile in LDS and its waves (one per token) also make the top-k selection.
// gridDim.z > 1: H is split over gridDim.z workgroups too (split blockIdx.z * n_splits + wave);
// each writes its partial tile, without the bias, to partials[blockIdx.z][T][E] instead of
// logits (not with SELECT).
// BATCH: 32-element steps whose loads go out together (one memory round trip per batch): 8 where
// 16 splits leave each wave about 6 steps, 12 where fewer splits leave it 12 or more (20B-shaped
// router, T = 8192: 40 -> 34 us; 12 with 16 splits only adds masked re-reads, 15 -> 18 us).
template <bool SELECT, int BATCH>
__global__ __launch_bounds__(1024) void route_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ br,
    int T, int H, int E, int n_groups, int n_splits, float* __restrict__ logits, int k,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, float* __restrict__ partials,
    int32_t* __restrict__ zero_word) {
  __shared__ float part[16][kTokPerWG][16];  // per wave: its partial 16 x 16 tile
  __shared__ float tile[SELECT ? kTokPerWG : 1][SELECT ? 257 : 1];  // the workgroup's logits
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * kTokPerWG;
  const int m = lane & 15, g = lane >> 4;
  const int gl = wave % n_groups, split = wave / n_groups;
  const int grp = blockIdx.y * n_groups + gl;
  // (a counter of the next launch, which starts from zero)
  if (zero_word != nullptr && blockIdx.x + blockIdx.y + blockIdx.z == 0 && threadIdx.x == 0) *zero_word = 0;

  // ---- partial logits: experts [16*grp, 16*grp + 16), 32-element steps [s0, s1) of H ----
  const int nsteps = H >> 5;
  const int all_splits = n_splits * gridDim.z, gsplit = blockIdx.z * n_splits + split;
  const int s0 = nsteps * gsplit / all_splits;
  const int s1 = nsteps * (gsplit + 1) / all_splits;
  f32x4 acc = logit_tile_partial<BATCH>(x, wr, T, H, E, t0, grp * 16, s0, s1, lane);
  // every split's tile goes to LDS; the first split of each group sums them in split order
  if (n_splits > 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][4 * g + i][m] = acc[i];
    __syncthreads();
    if (split == 0)
      for (int sp = 1; sp < n_splits; ++sp)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += part[sp * n_groups + gl][4 * g + i][m];
  }
  if (split == 0 && gridDim.z > 1) {
    const int e = grp * 16 + m;
    if (e < E) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * g + i;
        if (t < T) partials[((int64_t)blockIdx.z * T + t) * E + e] = acc[i];
      }
    }
  } else if (split == 0) {
    const int e = grp * 16 + m;
    if (e < E) {
      const float bias = (br != nullptr) ? br[e] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * g + i;
        if (t < T && logits != nullptr) logits[(int64_t)t * E + e] = acc[i] + bias;
        if constexpr (SELECT) tile[4 * g + i][e] = acc[i] + bias;
      }
    }
  }
  if constexpr (SELECT) {
    __syncthreads();
    const int nwaves = blockDim.x >> 6;  // n_groups * n_splits, at least 1
    for (int tt = wave; tt < kTokPerWG && t0 + tt < T; tt += nwaves)
      select_topk_wave([&](int e) { return tile[tt][e]; }, lane, t0 + tt, E, k, idx_out, w_out);
  }
}

// One 16-lane row per token (16 tokens per workgroup), logits read back from memory; with
// NP > 0 partial tiles, the row first sums partials[0..NP)[t][e] in that order, adds the bias and
// writes the logits (a compile-time NP lets all of a lane's loads go out together). NQ: experts
// per lane (E <= 16 NQ). Returns the row's logits (-inf past E).
template <int NQ, int NP>
__device__ __forceinline__ void select_row_logits(float* __restrict__ logits, int T, int E, int t,
                                                  int j16, const float* __restrict__ partials,
                                                  const float* __restrict__ br, float (&cv)[NQ]) {
  if constexpr (NP == 0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = j16 + 16 * q;
      cv[q] = (e < E) ? logits[(int64_t)t * E + e] : -INFINITY;
    }
  } else {
    float part[NP][NQ];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int e = min(j16 + 16 * q, E - 1);
        part[p][q] = partials[((int64_t)p * T + t) * E + e];
      }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = j16 + 16 * q;
      float s = part[0][q];
#pragma unroll
      for (int p = 1; p < NP; ++p) s += part[p][q];
      s += (br != nullptr) ? br[min(e, E - 1)] : 0.f;
      if (e < E) logits[(int64_t)t * E + e] = s;
      cv[q] = (e < E) ? s : -INFINITY;
    }
  }
}

template <int NQ, int NP>
__global__ __launch_bounds__(256) void route_select_kernel(float* __restrict__ logits, int T, int E,
                                                           int k, int32_t* __restrict__ idx_out,
                                                           float* __restrict__ w_out,
                                                           const float* __restrict__ partials,
                                                           const float* __restrict__ br) {
  const int j16 = threadIdx.x & 15;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (t >= T) return;
  float cv[NQ];
  select_row_logits<NQ, NP>(logits, T, E, t, j16, partials, br, cv);
  select_topk_row16<NQ>(cv, j16, t, E, k, idx_out, w_out);
}

// Decode-sized batches inside the MoE call: route_select_kernel's selection and then, by the
// workgroup that finishes its tokens last, the permutation of all pairs (one launch instead of
// two). Each workgroup stores its tokens' experts and weights device-coherent (written through
// to the device's point of coherence), waits until those stores are done and counts itself in
// on a counter the router launch set to zero; the one that counts last reads every pair's expert
// device-coherent and runs the permutation kernel's counting sort with its four waves.
template <int NQ, int NP>
__global__ __launch_bounds__(256) void route_select_permute_kernel(
    float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, const float* __restrict__ partials, const float* __restrict__ br,
    int32_t* __restrict__ counter, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int32_t* __restrict__ status, int32_t* __restrict__ dev_err,
    int tile_rows, int2* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  __shared__ int cnt[4][kPermuteMaxE];
  __shared__ int tot[kPermuteMaxE + 1];
  __shared__ int tbase[kPermuteMaxE + 1];
  __shared__ int bad, last;
  const int j16 = threadIdx.x & 15;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (t < T) {
    float cv[NQ];
    select_row_logits<NQ, NP>(logits, T, E, t, j16, partials, br, cv);
    select_topk_row16<NQ, true>(cv, j16, t, E, k, idx_out, w_out);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's stores are done
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (int)gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  permute_pairs<4>([&](int p) { return __hip_atomic_load(idx_out + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); },
                   T * k, E, offsets, perm, inv, status, dev_err, tile_rows, tiles, num_tiles,
                   &cnt[0][0], tot, tbase, &bad);
}

template <int NP>
void launch_select_np(int nq, dim3 grid, float* logits, int T, int E, int k, int32_t* idx, float* w,
                      const float* partials, const float* br, hipStream_t stream) {
  const dim3 block(256);
  if (nq <= 1) hipLaunchKernelGGL((route_select_kernel<1, NP>), grid, block, 0, stream, logits, T, E, k, idx, w, partials, br);
  else if (nq <= 2) hipLaunchKernelGGL((route_select_kernel<2, NP>), grid, block, 0, stream, logits, T, E, k, idx, w, partials, br);
  else if (nq <= 4) hipLaunchKernelGGL((route_select_kernel<4, NP>), grid, block, 0, stream, logits, T, E, k, idx, w, partials, br);
  else if (nq <= 8) hipLaunchKernelGGL((route_select_kernel<8, NP>), grid, block, 0, stream, logits, T, E, k, idx, w, partials, br);
  else hipLaunchKernelGGL((route_select_kernel<16, NP>), grid, block, 0, stream, logits, T, E, k, idx, w, partials, br);
}

// n_part: 0 (logits complete) or 2, 4, 8 partial tiles.
hipError_t launch_route_select(float* logits, int T, int E, int k, int32_t* idx, float* w,
                               const float* partials, int n_part, const float* br,
                               hipStream_t stream) {
  const dim3 grid((T + 15) / 16);
  const int nq = (E + 15) / 16;
  switch (n_part) {
    case 0: launch_select_np<0>(nq, grid, logits, T, E, k, idx, w, partials, br, stream); break;
    case 2: launch_select_np<2>(nq, grid, logits, T, E, k, idx, w, partials, br, stream); break;
    case 4: launch_select_np<4>(nq, grid, logits, T, E, k, idx, w, partials, br, stream); break;
    case 8: launch_select_np<8>(nq, grid, logits, T, E, k, idx, w, partials, br, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NP>
void launch_select_permute_np(int nq, dim3 grid, float* logits, int T, int E, int k, int32_t* idx,
                              float* w, const float* partials, const float* br, int32_t* counter,
                              int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* status,
                              int32_t* dev_err, int tile_rows, int2* tiles, int32_t* num_tiles,
                              hipStream_t stream) {
  const dim3 block(256);
#define MX_SP_LAUNCH(Q)                                                                           \
  hipLaunchKernelGGL((route_select_permute_kernel<Q, NP>), grid, block, 0, stream, logits, T, E, k, \
                     idx, w, partials, br, counter, offsets, perm, inv, status, dev_err,           \
                     tile_rows, tiles, num_tiles)
  if (nq <= 1) MX_SP_LAUNCH(1);
  else if (nq <= 2) MX_SP_LAUNCH(2);
  else if (nq <= 4) MX_SP_LAUNCH(4);
  else if (nq <= 8) MX_SP_LAUNCH(8);
  else MX_SP_LAUNCH(16);
#undef MX_SP_LAUNCH
}

// ---- large batches: 64-token tiles over all experts, staged through LDS ----
constexpr int kTileTok = 64;  // tokens per workgroup
constexpr int kTileK = 64;    // elements of H per stage: one 128-byte row per token / expert

template <int NB, int NW>  // 16-expert blocks (E <= 16 NB); waves (4, or 8: two per token group)
struct RouteTile {
  static constexpr int ROWS = kTileTok + 16 * NB;    // LDS rows per stage: tokens, then experts
  static constexpr int STAGE = ROWS * 128;            // bytes
  static constexpr int STAGES = NB >= 16 ? 3 : NB >= 8 ? 4 : 6;
  static constexpr int INSTR = ROWS / 8;              // 64 x 16-byte loads fill 8 rows
  static constexpr int PW = (INSTR + NW - 1) / NW;    // loads per wave and stage
  static constexpr int NBW = NB * 4 / NW;             // expert blocks per wave
  static_assert((STAGES - 2) * PW < 64, "vmcnt range");
  static_assert(NW == 4 || (NW == 8 && NB >= 2), "wave layout");
};

// Workgroup (blockIdx.x, blockIdx.y): tokens [64 bx, 64 bx + 64) x all experts over the
// 64-element chunks [c0, c1) of H that split by owns. Each stage holds the tile's 64 token rows
// and 16 NB expert rows (rows past T or E read as zeros) as 128-byte rows, chunks XOR-swizzled by
// row. Wave w computes tokens 16 (w % 4) .. + 15 against expert blocks [w / 4 * NBW, + NBW) (all
// of them with four waves; half with eight, two waves per SIMD). With one split the logits (plus
// the bias) go to logits, else the partial sums to partials[by][T][E].
template <int NB, int NW>
__global__ __launch_bounds__(64 * NW) void route_tile_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ wr,
                                                         const float* __restrict__ br, int T, int H,
                                                         int E, float* __restrict__ logits,
                                                         float* __restrict__ partials) {
  using RT = RouteTile<NB, NW>;
  __shared__ __align__(1024) uint8_t smem[RT::STAGES * RT::STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * kTileTok;
  const int nc = H / kTileK, S = gridDim.y;
  const int c0 = nc * (int)blockIdx.y / S, c1 = nc * ((int)blockIdx.y + 1) / S, n = c1 - c0;
  const i32x4 rx = make_res(x, (int64_t)T * H * 2);
  const i32x4 rw = make_res(wr, (int64_t)E * H * 2);

  // lane offsets of this wave's loads (fixed over the stages; chunk j adds 128 j bytes)
  uint32_t voff[RT::PW];
  int ldst[RT::PW];
#pragma unroll
  for (int q = 0; q < RT::PW; ++q) {
    const int i = (wave * RT::PW + q) % RT::INSTR;
    const int row = 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ swz_rows<8>(row);
    const int src = row < kTileTok ? t0 + row : row - kTileTok;
    const bool ok = row < kTileTok ? src < T : src < E;
    voff[q] = ok ? (uint32_t)src * (uint32_t)(H * 2) + 16u * c + 128u * c0 : kOutOfRange;
    ldst[q] = 1024 * i;
  }
  auto issue = [&](int j) {
    uint8_t* st = smem + (j % RT::STAGES) * RT::STAGE;
#pragma unroll
    for (int q = 0; q < RT::PW; ++q) {
      const bool is_x = __builtin_amdgcn_readfirstlane(ldst[q]) < kTileTok * 128;
      dma_b128(is_x ? rx : rw, off_add(voff[q], 128u * j), 0, st + ldst[q]);
    }
  };

  f32x4 acc[RT::NBW];
#pragma unroll
  for (int b = 0; b < RT::NBW; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int m = lane & 15, g = lane >> 4;
  const int tg = wave & 3, b0 = (wave >> 2) * RT::NBW;
  const int ar = 16 * tg + m;

#pragma unroll
  for (int j = 0; j < RT::STAGES - 1; ++j)
    if (j < n) issue(j);
  for (int j = 0; j < n; ++j) {
    if (j + RT::STAGES - 1 <= n) wait_vmcnt<(RT::STAGES - 2) * RT::PW>();
    else wait_vmcnt<0>();
    barrier_lds();
    if (j + RT::STAGES - 1 < n) issue(j + RT::STAGES - 1);
    const uint8_t* st = smem + (j % RT::STAGES) * RT::STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = 4 * ks + g;
      const u32x4 a = lds_read_b128(st + ar * 128 + ((ch ^ swz_rows<8>(ar)) << 4));
#pragma unroll
      for (int b = 0; b < RT::NBW; ++b) {
        const int r = kTileTok + 16 * (b0 + b) + m;
        const u32x4 w = lds_read_b128(st + r * 128 + ((ch ^ swz_rows<8>(r)) << 4));
        acc[b] = mfma16x16x32(u32x4_as_bf16x8(a), u32x4_as_bf16x8(w), acc[b]);
      }
    }
  }

  // value i of acc[b] in lane (m, g): token 16 tg + 4 g + i, expert 16 (b0 + b) + m
#pragma unroll
  for (int b = 0; b < RT::NBW; ++b) {
    const int e = 16 * (b0 + b) + m;
    if (e >= E) continue;
    const float bias = (S == 1 && br != nullptr) ? br[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * tg + 4 * g + i;
      if (t >= T) continue;
      if (S == 1) logits[(int64_t)t * E + e] = acc[b][i] + bias;
      else partials[((int64_t)blockIdx.y * T + t) * E + e] = acc[b][i];
    }
  }
}

// Splits of H per 64-token tile: doubled (to at most 8, each split at least two chunks) while
// the launch has fewer than 256 workgroups.
int route_tile_splits(int T, int H) {
  const int tiles = (T + kTileTok - 1) / kTileTok, nc = H / kTileK;
  int S = 1;
  while (S < 8 && tiles * S < 256 && nc >= 4 * S) S *= 2;
  return S;
}

// The tiled router applies to large batches (the ones the 16-token kernel runs with every expert
// group in one workgroup) whose H is a multiple of 64.
bool route_tiled(int T, int H, int E) {
  const int groups = (E + 15) / 16, tiles = (T + kTokPerWG - 1) / kTokPerWG;
  return H % kTileK == 0 && tiles * groups > kSpreadBelow;
}

hipError_t launch_route_tile(const uint16_t* x, const uint16_t* wr, const float* br, int T, int H,
                             int E, float* logits, float* partials, int S, hipStream_t stream) {
  const dim3 grid((T + kTileTok - 1) / kTileTok, S), b4(256), b8(512);
  const int nb = (E + 15) / 16;
  if (nb <= 1) hipLaunchKernelGGL((route_tile_kernel<1, 4>), grid, b4, 0, stream, x, wr, br, T, H, E, logits, partials);
  else if (nb <= 2) hipLaunchKernelGGL((route_tile_kernel<2, 8>), grid, b8, 0, stream, x, wr, br, T, H, E, logits, partials);
  else if (nb <= 4) hipLaunchKernelGGL((route_tile_kernel<4, 8>), grid, b8, 0, stream, x, wr, br, T, H, E, logits, partials);
  else if (nb <= 8) hipLaunchKernelGGL((route_tile_kernel<8, 8>), grid, b8, 0, stream, x, wr, br, T, H, E, logits, partials);
  else hipLaunchKernelGGL((route_tile_kernel<16, 8>), grid, b8, 0, stream, x, wr, br, T, H, E, logits, partials);
  return hipGetLastError();
}

// Workgroups per token tile and expert group in the spread launch, when partial sums have a
// buffer: doubled (up to 4) while the launch stays within 256 workgroups (20B-shaped router,
// T = 64: 8 tiles, 17 -> 12 us with 4; 120B-shaped, T = 256: 128 tiles, 17.5 -> 14 us with 2).
int route_spread_splits(int T, int H, int E) {
  const int groups = (E + 15) / 16, tiles = (T + kTokPerWG - 1) / kTokPerWG;
  const int base = tiles * groups;
  if (base > kSpreadBelow || H / 32 < 16) return 1;
  int so = 1;
  while (so < 4 && base * so * 2 <= 256) so *= 2;
  return so;
}

}  // namespace

// At most one token per wave of the permutation workgroup: with more, the selections queue up on
// its four SIMDs and cost more than the launch saved (20B-shaped decode, T = 64: the permutation
// launch grew from 7 to 27 us with the logits staged in LDS, against 5.5 us for the selection
// launch it replaced).
bool route_logits_defers_select(int T, int E, int k) {
  const int groups = (E + 15) / 16, tiles = (T + kTokPerWG - 1) / kTokPerWG;
  return groups > 1 && tiles * groups <= kSpreadBelow && T <= 16 && (int64_t)T * k <= kSelectMaxPairs &&
         (int64_t)T * E <= kSelectMaxLogits;
}

int route_partial_splits(int T, int H, int E) {
  return route_tiled(T, H, E) ? route_tile_splits(T, H) : route_spread_splits(T, H, E);
}

hipError_t launch_route_logits(const uint16_t* x, const uint16_t* wr, const float* br, int T,
                               int H, int E, float* logits, float* partials, int* n_part,
                               hipStream_t stream, int32_t* zero_word) {
  *n_part = 0;
  if (T == 0) return hipSuccess;
  const int groups = (E + 15) / 16, tiles = (T + kTokPerWG - 1) / kTokPerWG;
  const int splits = min(16, H / 32);
  // with a partials buffer H is also split over so workgroups per tile (splits is 16 then)
  const int so = partials != nullptr ? route_spread_splits(T, H, E) : 1;
  if (so > 1) *n_part = so;
  hipLaunchKernelGGL((route_logits_kernel<false, 8>), dim3(tiles, groups, so), dim3(64 * (splits / so)), 0,
                     stream, x, wr, br, T, H, E, 1, splits / so, logits, 0, nullptr, nullptr,
                     so > 1 ? partials : nullptr, zero_word);
  return hipGetLastError();
}

bool route_select_permute_fits(int T, int H, int E, int k) {
  const int groups = (E + 15) / 16, tiles = (T + kTokPerWG - 1) / kTokPerWG;
  return !route_logits_defers_select(T, E, k) && groups > 1 && tiles * groups <= kSpreadBelow &&
         !route_tiled(T, H, E) && (int64_t)T * k <= kSelectPermuteMaxPairs && E <= kPermuteMaxE;
}

hipError_t launch_route_select_permute(float* logits, const float* partials, int n_part,
                                       const float* br, int T, int E, int k, int32_t* idx,
                                       float* w, int32_t* counter, int32_t* offsets, int32_t* perm,
                                       int32_t* inv, int32_t* status, int tile_rows, int2* tiles,
                                       int32_t* num_tiles, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 15) / 16);
  const int nq = (E + 15) / 16;
  int32_t* dev_err = device_error_word();
  switch (n_part) {
    case 0: launch_select_permute_np<0>(nq, grid, logits, T, E, k, idx, w, partials, br, counter, offsets, perm, inv, status, dev_err, tile_rows, tiles, num_tiles, stream); break;
    case 2: launch_select_permute_np<2>(nq, grid, logits, T, E, k, idx, w, partials, br, counter, offsets, perm, inv, status, dev_err, tile_rows, tiles, num_tiles, stream); break;
    case 4: launch_select_permute_np<4>(nq, grid, logits, T, E, k, idx, w, partials, br, counter, offsets, perm, inv, status, dev_err, tile_rows, tiles, num_tiles, stream); break;
    case 8: launch_select_permute_np<8>(nq, grid, logits, T, E, k, idx, w, partials, br, counter, offsets, perm, inv, status, dev_err, tile_rows, tiles, num_tiles, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_route_topk(const uint16_t* x, const uint16_t* wr, const float* br, int T, int H,
                             int E, int k, float* logits, int32_t* idx, float* w, float* partials,
                             hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (logits != nullptr && route_tiled(T, H, E)) {
    const int S = route_tile_splits(T, H);
    if (S == 1 || partials != nullptr) {
      hipError_t e = launch_route_tile(x, wr, br, T, H, E, logits, partials, S, stream);
      if (e != hipSuccess) return e;
      return launch_route_select(logits, T, E, k, idx, w, partials, S > 1 ? S : 0, br, stream);
    }
  }
  const int groups = (E + 15) / 16, tiles = (T + kTokPerWG - 1) / kTokPerWG;
  // G groups per workgroup, H split so that G x splits fills up to 16 waves. Without a logits
  // buffer every workgroup covers all experts of its tokens and selects from LDS.
  const int G = (tiles * groups <= kSpreadBelow && logits != nullptr) ? 1 : groups;
  const int splits = min(16 / G, H / 32);
  if (G == groups) {  // one workgroup covers all experts of its tokens: select in the same kernel
    if (splits >= 16)
      hipLaunchKernelGGL((route_logits_kernel<true, 8>), dim3(tiles, 1), dim3(64 * G * splits), 0, stream,
                         x, wr, br, T, H, E, G, splits, logits, k, idx, w, nullptr, nullptr);
    else
      hipLaunchKernelGGL((route_logits_kernel<true, 12>), dim3(tiles, 1), dim3(64 * G * splits), 0, stream,
                         x, wr, br, T, H, E, G, splits, logits, k, idx, w, nullptr, nullptr);
    return hipGetLastError();
  }
  // (G is 1 here: one expert group per workgroup; splits is 16 wherever so > 1)
  const int so = partials != nullptr ? route_spread_splits(T, H, E) : 1;
  hipLaunchKernelGGL((route_logits_kernel<false, 8>), dim3(tiles, groups, so), dim3(64 * (splits / so)), 0,
                     stream, x, wr, br, T, H, E, 1, splits / so, logits, k, idx, w, partials, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_route_select(logits, T, E, k, idx, w, partials, so > 1 ? so : 0, br, stream);
}

}  // namespace mx
