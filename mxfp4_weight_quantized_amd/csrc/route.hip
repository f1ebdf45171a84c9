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
// wave per token (adds up the partial tiles and the bias first, if there are partials) ranks the
// logits (wave-wide argmax k times) and writes the top-k indices and their softmax.
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
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, float* __restrict__ partials) {
  __shared__ float part[16][kTokPerWG][16];  // per wave: its partial 16 x 16 tile
  __shared__ float tile[SELECT ? kTokPerWG : 1][SELECT ? 257 : 1];  // the workgroup's logits
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * kTokPerWG;
  const int m = lane & 15, g = lane >> 4;
  const int gl = wave % n_groups, split = wave / n_groups;
  const int grp = blockIdx.y * n_groups + gl;

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

// One wave per token, logits read back from memory; with n_part > 0 partial tiles, the wave
// first sums partials[0..n_part)[t][e] in that order, adds the bias and writes the logits.
__global__ __launch_bounds__(256) void route_select_kernel(float* __restrict__ logits, int T, int E,
                                                           int k, int32_t* __restrict__ idx_out,
                                                           float* __restrict__ w_out,
                                                           const float* __restrict__ partials,
                                                           int n_part, const float* __restrict__ br) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (n_part == 0) {
    select_topk_wave([&](int e) { return logits[(int64_t)t * E + e]; }, lane, t, E, k, idx_out, w_out);
    return;
  }
  select_topk_wave(
      [&](int e) {
        float s = partials[(int64_t)t * E + e];
        for (int p = 1; p < n_part; ++p) s += partials[((int64_t)p * T + t) * E + e];
        s += (br != nullptr) ? br[e] : 0.f;
        logits[(int64_t)t * E + e] = s;
        return s;
      },
      lane, t, E, k, idx_out, w_out);
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

// Workgroups per token tile and expert group in the spread launch, when partial sums have a
// buffer: doubled (up to 4) while the launch stays within 256 workgroups (20B-shaped router,
// T = 64: 8 tiles, 17 -> 12 us with 4; 120B-shaped, T = 256: 128 tiles, 17.5 -> 14 us with 2).
int route_partial_splits(int T, int H, int E) {
  const int groups = (E + 15) / 16, tiles = (T + kTokPerWG - 1) / kTokPerWG;
  const int base = tiles * groups;
  if (base > kSpreadBelow || H / 32 < 16) return 1;
  int so = 1;
  while (so < 4 && base * so * 2 <= 256) so *= 2;
  return so;
}

hipError_t launch_route_logits(const uint16_t* x, const uint16_t* wr, const float* br, int T,
                               int H, int E, float* logits, float* partials, int* n_part,
                               hipStream_t stream) {
  *n_part = 0;
  if (T == 0) return hipSuccess;
  const int groups = (E + 15) / 16, tiles = (T + kTokPerWG - 1) / kTokPerWG;
  const int splits = min(16, H / 32);
  // with a partials buffer H is also split over so workgroups per tile (splits is 16 then)
  const int so = partials != nullptr ? route_partial_splits(T, H, E) : 1;
  if (so > 1) *n_part = so;
  hipLaunchKernelGGL((route_logits_kernel<false, 8>), dim3(tiles, groups, so), dim3(64 * (splits / so)), 0,
                     stream, x, wr, br, T, H, E, 1, splits / so, logits, 0, nullptr, nullptr,
                     so > 1 ? partials : nullptr);
  return hipGetLastError();
}

hipError_t launch_route_topk(const uint16_t* x, const uint16_t* wr, const float* br, int T, int H,
                             int E, int k, float* logits, int32_t* idx, float* w, float* partials,
                             hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int groups = (E + 15) / 16, tiles = (T + kTokPerWG - 1) / kTokPerWG;
  // G groups per workgroup, H split so that G x splits fills up to 16 waves. Without a logits
  // buffer every workgroup covers all experts of its tokens and selects from LDS.
  const int G = (tiles * groups <= kSpreadBelow && logits != nullptr) ? 1 : groups;
  const int splits = min(16 / G, H / 32);
  if (G == groups) {  // one workgroup covers all experts of its tokens: select in the same kernel
    if (splits >= 16)
      hipLaunchKernelGGL((route_logits_kernel<true, 8>), dim3(tiles, 1), dim3(64 * G * splits), 0, stream,
                         x, wr, br, T, H, E, G, splits, logits, k, idx, w, nullptr);
    else
      hipLaunchKernelGGL((route_logits_kernel<true, 12>), dim3(tiles, 1), dim3(64 * G * splits), 0, stream,
                         x, wr, br, T, H, E, G, splits, logits, k, idx, w, nullptr);
    return hipGetLastError();
  }
  // (G is 1 here: one expert group per workgroup; splits is 16 wherever so > 1)
  const int so = partials != nullptr ? route_partial_splits(T, H, E) : 1;
  hipLaunchKernelGGL((route_logits_kernel<false, 8>), dim3(tiles, groups, so), dim3(64 * (splits / so)), 0,
                     stream, x, wr, br, T, H, E, 1, splits / so, logits, k, idx, w, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_select_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k,
                     idx, w, partials, so > 1 ? so : 0, br);
  return hipGetLastError();
}

}  // namespace mx
