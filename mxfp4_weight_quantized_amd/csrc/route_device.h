// route_device.h -- device functions of the routing steps, shared by the per-step kernels
// (route.hip, permute.hip) and the single-launch decode pipeline (single.hip): a partial tile of
// router logits on bf16 MFMA, the top-k selection with the softmax over the selected logits, and
// the stable counting sort of the (token, slot) pairs by expert.
#pragma once
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

constexpr int kPermuteMaxE = 256;  // experts the counting sort handles

// A 32-bit store of a result other workgroups of the same launch read: plain, or (COH)
// device-coherent (written through to the device's point of coherence).
template <bool COH, class V>
__device__ __forceinline__ void st_out(V* p, V v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// ---- router logits ----
// Partial logits of tokens [t0, t0 + 16) x experts [e0, e0 + 16) over the 32-element steps
// [s0, s1) of H, on one wave: lane l gives A row t0 + l%16 and B row (expert) e0 + l%16, K group
// l/16; the result's value i of lane l is token t0 + 4*(l/16) + i, expert e0 + l%16 (rows past T
// or E repeat the last one; the caller drops them). BATCH steps' loads go out together (one
// memory round trip per batch); steps past s1 re-read the last step and are zeroed.
template <int BATCH>
__device__ __forceinline__ f32x4 logit_tile_partial(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ wr, int T, int H,
                                                    int E, int t0, int e0, int s0, int s1,
                                                    int lane) {
  const int m = lane & 15, g = lane >> 4;
  const int tok = min(t0 + m, T - 1);
  const int ex = min(e0 + m, E - 1);
  const uint16_t* xa = x + (int64_t)tok * H + g * 8;
  const uint16_t* wb = wr + (int64_t)ex * H + g * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int st = s0; st < s1; st += BATCH) {
    u32x4 a[BATCH], b[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int su = min(st + u, s1 - 1);
      a[u] = *reinterpret_cast<const u32x4*>(xa + 32 * su);
      b[u] = *reinterpret_cast<const u32x4*>(wb + 32 * su);
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const u32x4 av = (st + u < s1) ? a[u] : u32x4{0u, 0u, 0u, 0u};
      acc = mfma16x16x32(u32x4_as_bf16x8(av), u32x4_as_bf16x8(b[u]), acc);
    }
  }
  return acc;
}

// ---- top-k selection (router and the fused selection in the permutation) ----
// (value desc, index asc) ordering: true if (va, ia) ranks before (vb, ib).
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// One wave ranks the E logits of token t (logit_of(e) for e < E; lane l holds experts l, l+64,
// l+128, l+192): k rounds of a wave-wide argmax under (logit desc, expert index asc), then the
// softmax of the k selected logits; lane j < k writes entry j and returns its expert index.
template <class LogitOf, bool COH = false>
__device__ __forceinline__ int select_topk_wave(LogitOf logit_of, int lane, int t, int E, int k,
                                                int32_t* __restrict__ idx_out,
                                                float* __restrict__ w_out) {
  float cv[4];
  int ci[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    ci[q] = e;
    cv[q] = (e < E) ? logit_of(e) : -INFINITY;
  }
  bool used[4] = {false, false, false, false};
  float sel_v[8];
  int sel_i[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (!used[q] && ci[q] < E && (bi == 0x7fffffff || ranks_before(cv[q], ci[q], bv, bi))) {
        bv = cv[q];
        bi = ci[q];
      }
    // wave-wide best: DPP exchanges inside each 16-lane row (partners lane^1, lane^2, then the
    // mirrored lane in the half row and in the row), then the four rows' bests combined
    // uniformly from lanes 0, 16, 32 and 48
    auto take = [&](float ov, int oi) {
      if (oi != 0x7fffffff && (bi == 0x7fffffff || ranks_before(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    };
    auto dpp_step = [&](auto ctrl) {
      constexpr int C = decltype(ctrl)::value;
      const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), C, 0xf, 0xf, false));
      const int oi = __builtin_amdgcn_update_dpp(0, bi, C, 0xf, 0xf, false);
      take(ov, oi);
    };
    dpp_step(std::integral_constant<int, 0xb1>{});   // quad_perm [1,0,3,2]: lane ^ 1
    dpp_step(std::integral_constant<int, 0x4e>{});   // quad_perm [2,3,0,1]: lane ^ 2
    dpp_step(std::integral_constant<int, 0x141>{});  // row_half_mirror: 7 - lane in 8
    dpp_step(std::integral_constant<int, 0x140>{});  // row_mirror: 15 - lane in 16
#pragma unroll
    for (int row = 1; row < 4; ++row)
      take(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * row)),
           __builtin_amdgcn_readlane(bi, 16 * row));
    {  // row 0 last, so that every lane ends with the same (uniform) result
      const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
      const int i0 = __builtin_amdgcn_readlane(bi, 0);
      take(v0, i0);
    }
    sel_v[j] = bv;
    sel_i[j] = bi;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (ci[q] == bi) used[q] = true;
  }
  float sum = 0.f, mine = 0.f;
  int mine_i = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    const float ev = expf(sel_v[j] - sel_v[0]);
    sum += ev;
    if (lane == j) {
      mine = ev;
      mine_i = sel_i[j];
    }
  }
  if (lane < k) {
    st_out<COH>(idx_out + (int64_t)t * k + lane, mine_i);
    st_out<COH>(w_out + (int64_t)t * k + lane, mine / sum);
  }
  return mine_i;
}

// The same selection on one 16-lane row of a wave per token: lane j of the row holds the logits
// of experts j, j + 16, ..., j + 16 (NQ - 1) in cv (entries past E are ignored). The four DPP
// exchanges inside the row leave the row's best in every lane of it, so no step crosses rows.
// Every lane of the row calls it; row lane j < k writes entry j (COH: device-coherent, for a
// reader in another workgroup of the same launch). The softmax is the same arithmetic as
// select_topk_wave's.
template <int NQ, bool COH = false>
__device__ __forceinline__ void select_topk_row16(const float (&cv)[NQ], int j16, int t, int E,
                                                  int k, int32_t* __restrict__ idx_out,
                                                  float* __restrict__ w_out) {
  uint32_t used = 0;
  float sel_v[8];
  int sel_i[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = j16 + 16 * q;
      if (!((used >> q) & 1u) && e < E && (bi == 0x7fffffff || ranks_before(cv[q], e, bv, bi))) {
        bv = cv[q];
        bi = e;
      }
    }
    auto dpp_step = [&](auto ctrl) {
      constexpr int C = decltype(ctrl)::value;
      const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), C, 0xf, 0xf, false));
      const int oi = __builtin_amdgcn_update_dpp(0, bi, C, 0xf, 0xf, false);
      if (oi != 0x7fffffff && (bi == 0x7fffffff || ranks_before(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    };
    dpp_step(std::integral_constant<int, 0xb1>{});   // quad_perm [1,0,3,2]: lane ^ 1
    dpp_step(std::integral_constant<int, 0x4e>{});   // quad_perm [2,3,0,1]: lane ^ 2
    dpp_step(std::integral_constant<int, 0x141>{});  // row_half_mirror: 7 - lane in 8
    dpp_step(std::integral_constant<int, 0x140>{});  // row_mirror: 15 - lane in 16
    sel_v[j] = bv;
    sel_i[j] = bi;
    if ((bi & 15) == j16) used |= 1u << (bi >> 4);
  }
  float sum = 0.f, mine = 0.f;
  int mine_i = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    const float ev = expf(sel_v[j] - sel_v[0]);
    sum += ev;
    if (j16 == j) {
      mine = ev;
      mine_i = sel_i[j];
    }
  }
  if (j16 < k) {
    st_out<COH>(idx_out + (int64_t)t * k + j16, mine_i);
    st_out<COH>(w_out + (int64_t)t * k + j16, mine / sum);
  }
}

// ---- stable counting sort of the (token, slot) pairs by expert ----
// Exclusive scan of n (<= 256) ints in LDS by one wave; returns the total to every lane.
__device__ __forceinline__ int wave_exclusive_scan(int* v, int n, int lane) {
  int carry = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const int x = (i < n) ? v[i] : 0;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (i < n) v[i] = carry + incl - x;
    carry += __shfl(incl, 63);
  }
  return carry;
}

// One workgroup of NW waves sorts the P pairs (expert of pair p: pair_expert(p)) by expert, with
// no global atomics: pair p belongs to wave p / C (C = ceil(P / NW)), each wave counts its chunk
// per expert in LDS, a scan over (expert, wave) gives every (wave, expert) its first output row,
// and each wave then scatters its chunk 64 pairs at a time, ranking equal experts among the 64
// lanes with ballots -- the stable (token, slot) order, so the result is deterministic. Writes
// offsets [E+1], perm [P], inv [P] (-1 for an index outside [0, E), which also sets *status = 1
// and the routing bit of dev_err), and with tile_rows > 0 the tile list and its length (perm then
// holds tile_rows entries of padding past P, set to pair 0 like the rows past the last valid
// pair). LDS from the caller: cnt [NW][kPermuteMaxE], tot and tbase [kPermuteMaxE + 1], bad [1].
// Every thread of the workgroup calls it. COH: the outputs are stored device-coherent.
// tile_ends (optional, with the tile list): each tile's expert's end row, offsets[e + 1].
template <int NW, class PairExpert, bool COH = false>
__device__ __forceinline__ void permute_pairs(PairExpert pair_expert, int P, int E,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                              int32_t* __restrict__ status,
                                              int32_t* __restrict__ dev_err, int tile_rows,
                                              int2* __restrict__ tiles,
                                              int32_t* __restrict__ num_tiles, int* cnt, int* tot,
                                              int* tbase, int* bad,
                                              int32_t* __restrict__ tile_ends = nullptr) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int chunk = (P + NW - 1) / NW;
  const int p_begin = min(P, wave * chunk);
  const int p_end = min(P, p_begin + chunk);
  int* my_cnt = cnt + wave * kPermuteMaxE;

  for (int i = threadIdx.x; i < NW * kPermuteMaxE; i += blockDim.x) cnt[i] = 0;
  if (threadIdx.x == 0) *bad = 0;
  __syncthreads();

  // 1. per-wave histogram
  for (int p = p_begin + lane; p < p_end; p += 64) {
    const int e = pair_expert(p);
    if (e >= 0 && e < E) atomicAdd(&my_cnt[e], 1);
    else *bad = 1;
  }
  __syncthreads();

  // 2. totals per expert, scan -> offsets; first row of every (wave, expert)
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int w = 0; w < NW; ++w) s += cnt[w * kPermuteMaxE + e];
    tot[e] = s;
    if (tile_rows > 0) tbase[e] = (s + tile_rows - 1) / tile_rows;
  }
  __syncthreads();
  if (wave == 0) {
    const int total = wave_exclusive_scan(tot, E, lane);
    if (lane == 0) tot[E] = total;
  } else if (wave == 1 && tile_rows > 0) {
    const int total = wave_exclusive_scan(tbase, E, lane);
    if (lane == 0) tbase[E] = total;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) st_out<COH>(offsets + e, tot[e]);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = tot[e];
    for (int w = 0; w < NW; ++w) {
      const int c = cnt[w * kPermuteMaxE + e];
      cnt[w * kPermuteMaxE + e] = run;
      run += c;
    }
    if (tile_rows > 0) {
      const int n = tot[e + 1] - tot[e];
      const int tb = tbase[e];
      for (int i = 0; i * tile_rows < n; ++i) {
        int* tl = reinterpret_cast<int*>(tiles + tb + i);
        st_out<COH>(tl, e);
        st_out<COH>(tl + 1, tot[e] + i * tile_rows);
        if (tile_ends != nullptr) st_out<COH>(tile_ends + tb + i, tot[e + 1]);
      }
    }
  }
  if (threadIdx.x == 0) {
    if (tile_rows > 0) st_out<COH>(num_tiles, tbase[E]);
    if (status != nullptr) st_out<COH>(status, *bad);
    if (*bad && dev_err != nullptr) atomicOr(dev_err, kDevErrRouting);
  }
  if (tile_rows > 0)
    for (int i = tot[E] + threadIdx.x; i < P + tile_rows; i += blockDim.x) st_out<COH>(perm + i, 0);
  __syncthreads();

  // 3. stable scatter, 64 pairs per step in (token, slot) order
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int g0 = p_begin; g0 < p_end; g0 += 64) {
    const int p = g0 + lane;
    int e = (p < p_end) ? pair_expert(p) : -1;
    const bool ok = (e >= 0 && e < E);
    if (!ok) {
      if (p < p_end) st_out<COH>(inv + p, -1);
      e = 0;
    }
    uint64_t peers = __ballot(ok);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const int rank = __popcll(peers & lt_mask);
    int pos = 0;
    if (ok) pos = my_cnt[e] + rank;
    __builtin_amdgcn_wave_barrier();
    if (ok) {
      st_out<COH>(perm + pos, p);
      st_out<COH>(inv + p, pos);
      if (rank == 0) my_cnt[e] = pos + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace mx
