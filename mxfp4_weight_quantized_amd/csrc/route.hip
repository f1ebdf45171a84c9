// route.hip -- router logits, top-k expert selection and softmax over the selected experts.
//
// The GGUF page ("Hugging Face Transformers GGUF 지원", agentlenshq.com, section "ggml Metal 커널
// 통합") names a dedicated top-k kernel for MoE expert selection; the router itself is the
// library's reading: logits = x W_r^T + b, top-k by (logit desc, expert index asc), softmax over
// the k selected logits.
//
// One workgroup handles 16 tokens with up to 16 waves: the experts are split into groups of 16
// (one 16 x 16 logit tile each, bf16 MFMA with fp32 accumulate, operands read straight from
// global memory -- W_r is small and stays in L2) and, when there are few groups, the reduction
// over H is split across waves too. The per-split partial tiles meet in LDS and are summed in a
// fixed order, so the logits do not depend on timing. The waves then run the top-k for the 16
// tokens, one token per wave at a time, with wave-wide argmax reductions.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {
namespace {

constexpr int kTokPerWG = 16;

// (value desc, index asc) ordering: true if (va, ia) ranks before (vb, ib).
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(1024) void route_topk_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ br,
    int T, int H, int E, int k, int n_groups, int n_splits, float* __restrict__ logits,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  __shared__ float part[16][kTokPerWG][16];  // per wave: its partial 16 x 16 tile
  __shared__ float lg[kTokPerWG][257];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int t0 = blockIdx.x * kTokPerWG;
  const int m = lane & 15, g = lane >> 4;
  const int grp = wave % n_groups, split = wave / n_groups;

  // ---- partial logits: experts [16*grp, 16*grp + 16), 32-element steps [s0, s1) of H ----
  const int nsteps = H >> 5;
  const int s0 = (int)((int64_t)nsteps * split / n_splits);
  const int s1 = (int)((int64_t)nsteps * (split + 1) / n_splits);
  const int tok = min(t0 + m, T - 1);
  const int ex = min(grp * 16 + m, E - 1);
  const uint16_t* xa = x + (int64_t)tok * H + g * 8;
  const uint16_t* wb = wr + (int64_t)ex * H + g * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int st = s0;
  for (; st + 8 <= s1; st += 8) {  // eight steps' loads in flight per batch
    u32x4 a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a[u] = *reinterpret_cast<const u32x4*>(xa + 32 * (st + u));
      b[u] = *reinterpret_cast<const u32x4*>(wb + 32 * (st + u));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = mfma16x16x32(u32x4_as_bf16x8(a[u]), u32x4_as_bf16x8(b[u]), acc);
  }
  for (; st < s1; ++st) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(xa + 32 * st);
    const u32x4 b = *reinterpret_cast<const u32x4*>(wb + 32 * st);
    acc = mfma16x16x32(u32x4_as_bf16x8(a), u32x4_as_bf16x8(b), acc);
  }
  // a split's tile goes to LDS; the first split of each group sums all splits in split order
  if (n_splits > 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][4 * g + i][m] = acc[i];
    __syncthreads();
    if (split == 0)
      for (int sp = 1; sp < n_splits; ++sp)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += part[sp * n_groups + grp][4 * g + i][m];
  }
  if (split == 0) {
    const int e = grp * 16 + m;
    const float bias = (br != nullptr && e < E) ? br[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * g + i;
      const float v = acc[i] + bias;
      lg[row][e] = v;
      if (logits != nullptr && e < E && t0 + row < T) logits[(int64_t)(t0 + row) * E + e] = v;
    }
  }
  __syncthreads();

  // ---- top-k + softmax, one token per wave at a time ----
  for (int row = wave; row < kTokPerWG; row += nwaves) {
    const int t = t0 + row;
    if (t >= T) break;
    // each lane holds up to four candidates: experts lane, lane+64, lane+128, lane+192
    float cv[4];
    int ci[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      ci[q] = e;
      cv[q] = (e < E) ? lg[row][e] : -INFINITY;
    }
    bool used[4] = {false, false, false, false};
    float sel_v[8];
    int sel_i[8];
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (!used[q] && ci[q] < E && (bi == 0x7fffffff || ranks_before(cv[q], ci[q], bv, bi))) {
          bv = cv[q];
          bi = ci[q];
        }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (oi != 0x7fffffff && (bi == 0x7fffffff || ranks_before(ov, oi, bv, bi))) {
          bv = ov;
          bi = oi;
        }
      }
      sel_v[j] = bv;
      sel_i[j] = bi;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (ci[q] == bi) used[q] = true;
    }
    if (lane == 0) {
      float sum = 0.f;
      for (int j = 0; j < k; ++j) sum += expf(sel_v[j] - sel_v[0]);
      for (int j = 0; j < k; ++j) {
        idx_out[(int64_t)t * k + j] = sel_i[j];
        w_out[(int64_t)t * k + j] = expf(sel_v[j] - sel_v[0]) / sum;
      }
    }
  }
}

}  // namespace

hipError_t launch_route_topk(const uint16_t* x, const uint16_t* wr, const float* br, int T, int H,
                             int E, int k, float* logits, int32_t* idx, float* w,
                             hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // expert groups of 16; splits of H so that groups x splits fills up to 16 waves
  const int groups = (E + 15) / 16;
  const int splits = groups > 4 ? 1 : min(16 / groups, H / 32);
  const unsigned grid = (unsigned)((T + kTokPerWG - 1) / kTokPerWG);
  hipLaunchKernelGGL(route_topk_kernel, dim3(grid), dim3(64 * groups * splits), 0, stream, x, wr,
                     br, T, H, E, k, groups, splits, logits, idx, w);
  return hipGetLastError();
}

}  // namespace mx
