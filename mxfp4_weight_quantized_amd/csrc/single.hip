// single.hip -- the MoE MLP of a decode-sized batch as one persistent launch: router logits,
// top-k and softmax, the permutation by expert, the gate_up and down grouped GEMMs and the
// combine, with the dependencies between the steps resolved on the GPU instead of at kernel
// boundaries. The Korean GGUF page ("Hugging Face Transformers GGUF 지원", section "생성 루프
// 최적화") puts the cost of token generation in the synchronisation between the host and the GPU
// around each step; a decode-sized layer here is a chain of small dependent steps, and this form
// runs the chain without returning to the command processor between them.
//
// Work units, taken from device counters by whichever workgroups are running: first the routing
// units (with internal routing: token tile of 16 x expert group of 16 x H split -- a partial
// 16 x 16 tile of logits, bf16 MFMA with fp32 accumulate; with the caller's routing, one unit
// that sorts its pairs), then -- once the routing is done -- the gate_up tiles of every row tile
// and after them the down tiles. A unit only waits for units taken before it, by workgroups that
// are running them, and the units those wait for were taken earlier still, so every wait ends
// however many workgroups are resident. Hand-overs:
//   - the last routing unit of a token tile stages the tile's partial logits in LDS, sums them in
//     split order, adds the bias and makes the top-k selection and softmax of its tokens (the
//     router's function);
//   - the last token tile's selector (with one token tile: the same workgroup, from LDS) sorts
//     the pairs by expert (the permutation's function) and raises the routed flag, which carries
//     the number of row tiles;
//   - a down tile waits until every gate_up tile of its row tile is done;
//   - the last down tile of a column tile combines those columns for every token.
// The last workgroup to finish sets the counters back to zero for the next call, so calls on
// one device must not overlap (they share the counters). Each wait is bounded: past the spin
// limit it gives up, sets MX_DEVERR_SYNC in the device error word (the outputs are then not
// valid) and goes on; every load stays within its buffer either way.
//
// Measured against the per-step launches on the same layers, this form is slower (20B-shaped
// decode, T = 64: 140 vs 96 us; 120B-shaped, T = 1: 53 vs 39 us): the per-step launches' kernel
// boundaries are cheap here, and each hand-over inside the launch costs memory round trips on
// the critical path (a store written through, a counter, a poll), tile by tile.
#include "gemm_tile.h"
#include "route_device.h"

#include <atomic>

namespace mx {

// Counters of the single-launch pipeline, one array per device (zero at load; each call leaves
// it zero). Layout: routing-unit claims, selected token tiles, finished workgroups, GEMM-tile
// claims, the routed flag (1 + the number of row tiles, once the pairs are sorted), then per token
// tile (routing units done), per row tile (gate_up tiles done), per down column tile (down tiles
// done).
constexpr int kSingleMaxTokTiles = kSingleMaxPairs / 16;
constexpr int kSingleMaxRowTiles = kSingleMaxPairs / 16 + kPermuteMaxE;
constexpr int kSingleMaxColTiles = 3072 / 64;
// Each counter sits on its own 256-byte line, and the routed flag has kRoutedCopies copies that the
// waiting workgroups poll spread out: hundreds of workgroups polling one line had slowed the
// atomics of the routing units that share its memory channel several-fold.
constexpr int kRoutedCopies = 32;
enum : int { kSyClaimR = 0, kSySel = 1, kSyDone = 2, kSyClaimG = 3, kSyRouted = 4,
             kSyTok = kSyRouted + kRoutedCopies, kSyGu = kSyTok + kSingleMaxTokTiles,
             kSyDn = kSyGu + kSingleMaxRowTiles, kSyWords = kSyDn + kSingleMaxColTiles };
constexpr int kSyPad = 64;  // ints per counter line
__device__ int32_t g_single_sync[kSyWords * kSyPad];

namespace {

constexpr int kSpinLimit = 1 << 18;  // polls of about 1 us each: a wait gives up after ~0.3 s

struct SingleArgs {
  GemmKArgs gu, dn;
  const uint16_t* x;
  const uint16_t* wr;
  const float* br;
  int T, H, F, E, k, P;
  int route;           // 1: the routing units compute idx and w; 0: they are the caller's
  float* logits;       // [T][E] or null
  float* rpart;        // [r_splits][T][E] partial logits
  int r_splits;
  int32_t* idx;        // [T][k]
  float* w;            // [T][k]
  int32_t *offsets, *perm, *inv, *status, *num_tiles;
  int2* tiles;
  int32_t* tile_ends;  // [max_tiles] end row of each tile's expert
  int max_tiles;
  int nt_gu, nt_dn, bn_dn;
  const float* y;      // [P][H] down rows
  void* out;
  const float* dn_bias;
  int32_t* sync;
  int32_t* dev_err;
};

__device__ __forceinline__ int32_t* sy(const SingleArgs& a, int i) { return a.sync + i * kSyPad; }

// Every wave's memory operations so far have completed (stores written, loads returned).
__device__ __forceinline__ void wait_memory() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

// Hand-over between workgroups: whatever one workgroup leaves for others -- partial logits,
// selections, the sorted pairs, h, the down rows -- is stored device-coherent (written through
// to the device's point of coherence) and loaded device-coherent by the reader, so a hand-over
// needs only the writer's stores to have completed before its count moves: no L2 write-back at
// release or invalidation at acquire. (With them -- a release and an acquire fence per hand-over
// -- each fence wrote back or invalidated a whole XCD's L2 and the launch took 2-8x the separate
// launches' time.) Returns the count before the add, to every thread.
__device__ __forceinline__ int publish(int32_t* ctr, int* s_word, int add = 1) {
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) *s_word = __hip_atomic_fetch_add(ctr, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *s_word;
}

// Thread 0 polls *ctr until it reaches target (or the spin limit: error bit, then on); returns
// the count it saw, to every thread.
__device__ __forceinline__ int wait_count(const int32_t* ctr, int target, int32_t* dev_err,
                                          int* s_word) {
  if (threadIdx.x == 0) {
    int n = 0, v;
    while ((v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < target) {
      if (++n > kSpinLimit) {
        if (dev_err != nullptr) atomicOr(dev_err, kDevErrSync);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    *s_word = v;
  }
  __syncthreads();
  return *s_word;
}

// Row tile mt of the list: its expert, first row and the expert's end row (one round of loads),
// clamped into range.
__device__ __forceinline__ void row_tile(const SingleArgs& a, int mt, int& e, int& r0, int& row_end) {
  const int* tl = reinterpret_cast<const int*>(a.tiles + mt);
  const int e0 = ld_int<true>(tl), r00 = ld_int<true>(tl + 1), end0 = ld_int<true>(a.tile_ends + mt);
  e = __builtin_amdgcn_readfirstlane(min(max(e0, 0), a.E - 1));
  r0 = __builtin_amdgcn_readfirstlane(min(max(r00, 0), a.P));
  row_end = __builtin_amdgcn_readfirstlane(min(max(end0, r0), a.P));
}

template <bool BF16_OUT>
__device__ __forceinline__ void combine_columns(const SingleArgs& a, int c0) {
  const int c8 = (min(a.H, c0 + a.bn_dn) - c0) >> 3;
  for (int i = threadIdx.x; i < a.T * c8; i += blockDim.x)
    combine8<BF16_OUT, true>(a.y, a.inv, a.w, i / c8, c0 + (i % c8) * 8, a.H, a.k, a.P, a.out, a.idx,
                       a.dn_bias);
}

struct RouteLds {
  float part[4][16][16];
};
struct PermLds {
  int cnt[4][kPermuteMaxE];
  int tot[kPermuteMaxE + 1];
  int tbase[kPermuteMaxE + 1];
  int bad;
  int sidx[16 * 8];  // one token tile's selections (a batch of at most 16 tokens)
};

template <class T0, class T1, class T2, class T3>
constexpr size_t max_size() {
  size_t m = sizeof(T0);
  m = sizeof(T1) > m ? sizeof(T1) : m;
  m = sizeof(T2) > m ? sizeof(T2) : m;
  return sizeof(T3) > m ? sizeof(T3) : m;
}

// The routed flag, in every copy, once the sorted pairs are written: 1 + the number of row tiles.
__device__ __forceinline__ void raise_routed(const SingleArgs& a, const PermLds& pl) {
  wait_memory();
  __syncthreads();
  if (threadIdx.x < kRoutedCopies)
    __hip_atomic_store(sy(a, kSyRouted + threadIdx.x), 1 + pl.tbase[a.E], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// The pairs sorted by expert (one workgroup), then the routed flag.
__device__ __forceinline__ void permute_unit(const SingleArgs& a, PermLds& pl) {
  const int32_t* idx = a.idx;
  auto expert = [&](int p) { return ld_int<true>(idx + p); };
  permute_pairs<4, decltype(expert), true>(expert, a.P, a.E, a.offsets, a.perm, a.inv, a.status,
                                           a.dev_err, 16, a.tiles, a.num_tiles, &pl.cnt[0][0],
                                           pl.tot, pl.tbase, &pl.bad, a.tile_ends);
  raise_routed(a, pl);
}

// Routing unit u: a partial logit tile; the last unit of its token tile selects, the last
// selector permutes.
__device__ __forceinline__ void route_unit(const SingleArgs& a, int u, RouteLds& rl, PermLds& pl,
                                           float* stage, int* s_word) {
  const int S = a.r_splits, n_eg = (a.E + 15) / 16, n_tt = (a.T + 15) / 16;
  const int per_tt = n_eg * S;
  const int tt = u / per_tt, eg = (u % per_tt) / S, s = u % S;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  {
    const int nsteps = a.H >> 5, parts = 4 * S, q = 4 * s + wave;
    const f32x4 acc = logit_tile_partial<4>(a.x, a.wr, a.T, a.H, a.E, 16 * tt, 16 * eg,
                                            nsteps * q / parts, nsteps * (q + 1) / parts, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) rl.part[wave][4 * g + i][m] = acc[i];
  }
  __syncthreads();
  if (wave == 0) {
    const int e = 16 * eg + m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tt + 4 * g + i;
      const float v = rl.part[0][4 * g + i][m] + rl.part[1][4 * g + i][m] + rl.part[2][4 * g + i][m] +
                      rl.part[3][4 * g + i][m];
      if (t < a.T && e < a.E) st_out<true>(a.rpart + ((int64_t)s * a.T + t) * a.E + e, v);
    }
  }
  if (publish(sy(a, kSyTok + tt), s_word) != per_tt - 1) return;
  // selection of the tile's tokens, one wave per token: the splits' partial logits staged in LDS
  // with one round of loads, then summed in split order, plus the bias
  const int t0 = 16 * tt, nt_tok = min(a.T, t0 + 16) - t0, row = nt_tok * a.E;
  const int n_stage = S * row;  // at most 16 * 32 * 16 floats: (E / 16) * S <= 32
  {
    constexpr int kPer = 32;  // n_stage / 256 at most
    float v[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = threadIdx.x + 256 * r;
      v[r] = i < n_stage ? __hip_atomic_load(a.rpart + ((int64_t)(i / row) * a.T + t0) * a.E + i % row,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : 0.f;
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = threadIdx.x + 256 * r;
      if (i < n_stage) stage[i] = v[r];
    }
  }
  __syncthreads();
  const bool one_tile = n_tt == 1;  // then this workgroup sorts the pairs too, from LDS
  for (int tl = wave; tl < nt_tok; tl += 4) {
    const int t = t0 + tl;
    auto logit = [&](int e) {
      float v = stage[tl * a.E + e];
      for (int p = 1; p < S; ++p) v += stage[p * row + tl * a.E + e];
      v += (a.br != nullptr) ? a.br[e] : 0.f;
      if (a.logits != nullptr) a.logits[(int64_t)t * a.E + e] = v;
      return v;
    };
    const int ex = select_topk_wave<decltype(logit), true>(logit, lane, t, a.E, a.k, a.idx, a.w);
    if (one_tile && lane < a.k) pl.sidx[tl * a.k + lane] = ex;
  }
  if (one_tile) {
    __syncthreads();
    auto expert = [&](int p) { return pl.sidx[p]; };
    permute_pairs<4, decltype(expert), true>(expert, a.P, a.E, a.offsets, a.perm, a.inv, a.status,
                                             a.dev_err, 16, a.tiles, a.num_tiles, &pl.cnt[0][0],
                                             pl.tot, pl.tbase, &pl.bad, a.tile_ends);
    raise_routed(a, pl);
    return;
  }
  if (publish(sy(a, kSySel), s_word) != n_tt - 1) return;
  permute_unit(a, pl);
}

// CG, CD: the gate_up and down tile configurations (16-row tiles of four waves, resident scales).
template <class CG, class CD, bool TW, bool BF16_OUT>
__global__ __launch_bounds__(256, (CG::OCC * 4 + 3) / 4) void moe_single_launch_kernel(SingleArgs a) {
  static_assert(CG::BM == 16 && CD::BM == 16 && CG::WM * CG::WN == 4 && CD::WM * CD::WN == 4,
                "16-row tiles of four waves");
  static_assert(CG::SCM == SCM_RESIDENT && CD::SCM == SCM_RESIDENT, "resident scales");
  using LG = GemmLds<CG::BM, CG::BN, CG::WM, CG::WN, CG::KT, CG::ST, MODE_GATE_UP, false, CG::SCM, TW>;
  using LDn = GemmLds<CD::BM, CD::BN, CD::WM, CD::WN, CD::KT, CD::ST, MODE_DOWN, false, CD::SCM, TW>;
  constexpr size_t kBytes = max_size<typename LG::Storage, typename LDn::Storage, RouteLds, PermLds>();
  static_assert(sizeof(PermLds) + 16 * 32 * 16 * sizeof(float) <= kBytes, "selection staging");
  static_assert(kBytes * CG::OCC <= 160 * 1024, "LDS for the resident workgroups");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kBytes];
  __shared__ int s_word;
  auto& sg = *reinterpret_cast<typename LG::Storage*>(smem);
  auto& sd = *reinterpret_cast<typename LDn::Storage*>(smem);
  auto& rl = *reinterpret_cast<RouteLds*>(smem);
  auto& pl = *reinterpret_cast<PermLds*>(smem);
  float* stage = reinterpret_cast<float*>(smem + sizeof(PermLds));  // selection: partial logits

  const int n_tt = (a.T + 15) / 16, n_eg = (a.E + 15) / 16;
  const int u_route = a.route ? n_tt * n_eg * a.r_splits : 1;  // (or the one permutation unit)
  auto claim = [&](int which) {
    __syncthreads();  // the previous unit is done with the LDS and with s_word
    if (threadIdx.x == 0) s_word = __hip_atomic_fetch_add(sy(a, which), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return s_word;
  };
  // routing units (or the permutation of the caller's routing); none of them waits
  for (int u = claim(kSyClaimR); u < u_route; u = claim(kSyClaimR)) {
    if (a.route) route_unit(a, u, rl, pl, stage, &s_word);
    else permute_unit(a, pl);
  }
  // GEMM tiles, once the routing is done: the gate_up tiles of every row tile, then the down tiles
  const int routed = wait_count(sy(a, kSyRouted + blockIdx.x % kRoutedCopies), 1, a.dev_err, &s_word);
  const int ntiles = __builtin_amdgcn_readfirstlane(min(max(routed - 1, 0), a.max_tiles));
  const int n_gu = ntiles * a.nt_gu;
  const int n_all = n_gu + (ntiles > 0 ? ntiles * a.nt_dn : a.nt_dn);  // (no valid pair: zero output)
  for (int c = claim(kSyClaimG); c < n_all; c = claim(kSyClaimG)) {
    int e, r0, row_end;
    if (c < n_gu) {
      const int mt = c / a.nt_gu, nt = c % a.nt_gu;
      row_tile(a, mt, e, r0, row_end);
      gemm_tile<CG::BM, CG::BN, CG::WM, CG::WN, CG::KT, CG::ST, MODE_GATE_UP, false, CG::SCM, TW,
                CG::MF, true, true>(a.gu, sg, e, r0, row_end, nt);
      publish(sy(a, kSyGu + mt), &s_word);
      continue;
    }
    const int v = c - n_gu;
    if (ntiles == 0) {
      combine_columns<BF16_OUT>(a, v * a.bn_dn);
      continue;
    }
    const int mt = v / a.nt_dn, nt = v % a.nt_dn;
    wait_count(sy(a, kSyGu + mt), a.nt_gu, a.dev_err, &s_word);
    row_tile(a, mt, e, r0, row_end);
    gemm_tile<CD::BM, CD::BN, CD::WM, CD::WN, CD::KT, CD::ST, MODE_DOWN, false, CD::SCM, TW, CD::MF,
              true, true>(a.dn, sd, e, r0, row_end, nt);
    if (publish(sy(a, kSyDn + nt), &s_word) == ntiles - 1)
      combine_columns<BF16_OUT>(a, nt * a.bn_dn);
  }
  // the last workgroup out sets the counters back to zero for the next call
  __syncthreads();
  // (relaxed: every counter operation of this workgroup has returned before it counts itself out)
  if (threadIdx.x == 0) s_word = __hip_atomic_fetch_add(sy(a, kSyDone), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_word == (int)gridDim.x - 1)
    for (int i = threadIdx.x; i < kSyWords; i += blockDim.x)
      __hip_atomic_store(sy(a, i), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device address of the counters on the current device (nullptr if the lookup failed).
int32_t* single_sync_words() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int32_t*> addr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  int32_t* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* s = nullptr;
    if (hipGetSymbolAddress(&s, HIP_SYMBOL(g_single_sync)) != hipSuccess) return nullptr;
    p = static_cast<int32_t*>(s);
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

// Compute units of the current device (0 if the query failed), looked up once per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <class CG, class CD, bool TW, bool BF16_OUT>
hipError_t launch_single_kernel(const SingleArgs& a, hipStream_t stream) {
  // as many workgroups as the tile configuration is sized to keep resident per CU (the schedule
  // needs none of them to be resident for its waits to end)
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  hipLaunchKernelGGL((moe_single_launch_kernel<CG, CD, TW, BF16_OUT>), dim3((unsigned)(cus * CG::OCC)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <class CG, class CD, bool TW>
hipError_t launch_single(const SingleArgs& a, bool bf16_out, hipStream_t stream) {
  return bf16_out ? launch_single_kernel<CG, CD, TW, true>(a, stream)
                  : launch_single_kernel<CG, CD, TW, false>(a, stream);
}

}  // namespace

// H splits of the routing units: doubled while the launch has at most 512 of them, a token tile
// at most 32 (each adds one to the tile's counter), and every wave keeps at least two 32-element
// steps of H.
int single_route_splits(int T, int H, int E) {
  const int groups = (E + 15) / 16;
  const int base = ((T + 15) / 16) * groups;
  const int nsteps = H / 32;
  int S = 1;
  while (S < 16 && base * S * 2 <= 512 && groups * S * 2 <= 32 && nsteps >= 2 * 4 * (S * 2)) S *= 2;
  return S;
}

hipError_t launch_moe_single(const MoeGemmArgs& m, const SingleRouting& r, hipStream_t stream) {
  int32_t* sync = single_sync_words();
  if (sync == nullptr) return hipErrorInvalidSymbol;
  const bool tiny = use_tiny_tiles(m.T, m.k, m.E, 2 * m.F);
  SingleArgs a{};
  a.gu = gate_up_args(m);
  a.dn = down_args(m);
  a.x = m.x;
  a.wr = r.wr;
  a.br = r.br;
  a.T = m.T; a.H = m.H; a.F = m.F; a.E = m.E; a.k = m.k; a.P = m.T * m.k;
  a.route = r.wr != nullptr ? 1 : 0;
  a.logits = r.logits;
  a.rpart = r.rpart;
  a.r_splits = single_route_splits(m.T, m.H, m.E);
  a.idx = const_cast<int32_t*>(m.topk_idx);
  a.w = const_cast<float*>(m.topk_w);
  a.offsets = const_cast<int32_t*>(m.offsets);
  a.perm = const_cast<int32_t*>(m.perm);
  a.inv = const_cast<int32_t*>(m.inv);
  a.status = r.status;
  a.num_tiles = const_cast<int32_t*>(m.num_tiles);
  a.tiles = const_cast<int2*>(m.tiles);
  a.tile_ends = r.tile_ends;
  a.max_tiles = m.max_tiles;
  a.y = m.y;
  a.out = m.out;
  a.dn_bias = m.act_custom ? m.dn_bias : nullptr;
  a.sync = sync;
  a.dev_err = device_error_word();
  if (tiny) {
    a.nt_gu = (m.F + CfgTinyGU::BN / 2 - 1) / (CfgTinyGU::BN / 2);
    a.bn_dn = CfgTinyDn::BN;
  } else {
    a.nt_gu = (m.F + CfgDecGU::BN / 2 - 1) / (CfgDecGU::BN / 2);
    a.bn_dn = CfgDecDn128::BN;
  }
  a.nt_dn = (m.H + a.bn_dn - 1) / a.bn_dn;
  a.gu.n_tiles = a.nt_gu;
  a.dn.n_tiles = a.nt_dn;
  if (tiny)
    return m.tiled ? launch_single<CfgTinyGU, CfgTinyDn, true>(a, m.out_bf16, stream)
                   : launch_single<CfgTinyGU, CfgTinyDn, false>(a, m.out_bf16, stream);
  return m.tiled ? launch_single<CfgDecGU, CfgDecDn128, true>(a, m.out_bf16, stream)
                 : launch_single<CfgDecGU, CfgDecDn128, false>(a, m.out_bf16, stream);
}

}  // namespace mx
