// Fused decode path of the NVFP4 MoE layer, gfx950: S2-S6 of a few-token forward (T <= 32) in one
// launch after the router's, so the whole layer is two launches.  The pages' fastest sm_12x MoE
// is one fused kernel (token dispatch, the two GEMMs, SwiGLU and the top-k-weight reduction:
// "vLLM on the NVIDIA DGX Spark: A Complete Technical Guide", section 4, b12x), kept beside a
// separate small-batch micro path ("Serving Solar Open 2 on DGX Spark", "Adding Expert Parallelism
// to b12x"); at decode sizes the launch gaps and the short stage kernels leave HBM idle for a
// seventh of the pass, which this path removes.
//
// Work items, one per workgroup, in workgroup-index order:
//   0                       top-k of every token + the permutation, published with a release flag
//   shared gate/up tiles    need nothing but x
//   routed gate/up tiles    wait for the routing; from the lag-th routed m-tile on, each m-tile's
//                           gate/up tiles are followed by the down tiles of the m-tile `lag` places
//                           earlier (lag: about one GPU-full of gate/up tiles), so a down tile
//                           usually finds its rows of h complete when it starts
//   remaining down tiles    wait for the routing and the gate/up tiles of their m-tile
//   combine slices          wait for every down tile
// Every item waits only for items of smaller workgroup index.  The GPU dispatches the workgroups of
// a launch to each XCD in index order, so the producer of any wait has been dispatched before its
// consumer on its own XCD, or will be once that XCD's earlier workgroups -- none of which waits for a
// later one -- finish; each wait is also bounded (kSpinLimit polls), after which it records an error
// and the combine writes NaN rows instead of the output (a loud failure, never a hang).  The tiles are
// the skinny tiles of the stand-alone grouped GEMM (gemm_skinny.h) and the combine is
// combine_row.h, so results are bitwise those of the staged launches.
//
// Hand-offs: the tiles write h and y with device-coherent (agent-scope) stores, which reach memory
// past this XCD's L2; every wave waits for its stores, a workgroup barrier, then thread 0 increments
// the counter.  A consumer's thread 0 polls with agent-scope loads, then a barrier; the produced rows
// are read only after that, and no cache can hold an earlier copy of them, since nothing reads them
// before they are produced within the launch and every launch starts with clean caches.  The routing
// (written once, by plain stores) is published with a release fence (L2 write-back) and flag.  The
// counters live in the workspace and are cleared by the router launch of the same forward (no
// memset, no reliance on the caller's buffer contents), so the pair of launches can be captured in
// a HIP graph and replayed.
#include "combine_row.h"
#include "device_util.h"
#include "gemm_skinny.h"

namespace moe {
namespace {

// counter block (int32 words)
constexpr int kCtrReady = 1;    // 1 once the routing is published
constexpr int kCtrMtiles = 2;   // m-tiles that exist (shared + routed), published with the routing
constexpr int kCtrDnDone = 3;   // finished down tiles
constexpr int kCtrError = 4;    // a wait ran past its bound
constexpr int kCtrMtile0 = 8;   // per m-tile: finished gate/up n-tiles
constexpr int kSpinLimit = 1 << 20;
constexpr int kNB = 2;          // weight fragments per wave of the skinny tiles
constexpr int kWaves = kSkinnyThreads / kWave;
constexpr int kTokPerWave = kFusedDecodeMaxTokens / kWaves;

__device__ __forceinline__ int load_agent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 polls until *word >= target (or the bound runs out: error recorded); the barrier then
// holds every thread until then.  Called by the whole workgroup.
__device__ __forceinline__ void wg_wait_ge(const int32_t* word, int target, int32_t* err) {
  if (threadIdx.x == 0) {
    int v = load_agent(word);
    for (int it = 0; v < target; ++it) {
      if (it >= kSpinLimit) {
        __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
      v = load_agent(word);
    }
  }
  __syncthreads();
}

// The workgroup's device-coherent stores have completed (every wave waits for its stores before the
// barrier), then the increment.  Whole workgroup.
__device__ __forceinline__ void wg_signal(int32_t* word) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(word, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Layout {
  int xt;      // shared-expert m-tiles
  int mt_r;    // bound on routed m-tiles
  int nt_gu;   // gate/up n-tiles per m-tile
  int nt_dn;   // down n-tiles per m-tile
  int ncpt;    // combine slices per token
  int lag;     // routed m-tiles whose gate/up items precede the first routed down items
};

struct RouteLds {
  int ids[kFusedDecodeMaxSlots];
  int cnt[kFusedDecodeMaxExperts];
  int offs[kFusedDecodeMaxExperts];
  int mt;
};
template <int BKG, int BKD>
union FusedLds {
  SkinnyLds<BKG> g;
  SkinnyLds<BKD> d;
  RouteLds r;
};

// S2 + S3 by one workgroup: the top-k of every token (wave w takes tokens w, w + 4, ...; all of a
// wave's logits are loaded before its first selection), then the stable permutation of the T*k
// slots, then the release of the routing.
template <int VPL>
__device__ __forceinline__ void publish_routing(const FusedDecodeProblem& p, const Layout& y, RouteLds& r) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = p.T, E = p.E, k = p.k, S = T * k;
  float raw[kTokPerWave][VPL];
#pragma unroll
  for (int j = 0; j < kTokPerWave; ++j) {
    const int t = wave + kWaves * j;
    if (t < T) topk_load<VPL>(p.logits + (size_t)t * E, E, raw[j]);
  }
#pragma unroll
  for (int j = 0; j < kTokPerWave; ++j) {
    const int t = wave + kWaves * j;
    if (t < T) {
      int id;
      float wt;
      topk_select<VPL>(raw[j], E, k, &id, &wt);
      if (lane < k) {
        p.ids[(size_t)t * k + lane] = id;
        p.w[(size_t)t * k + lane] = wt;
        r.ids[t * k + lane] = id;
      }
    }
  }
  for (int e = tid; e < E; e += kSkinnyThreads) r.cnt[e] = 0;
  if (tid == 0) r.mt = 0;
  __syncthreads();
  for (int s = tid; s < S; s += kSkinnyThreads) atomicAdd(&r.cnt[r.ids[s]], 1);
  __syncthreads();
  if (wave == 0) {
    const int total = wave_exclusive_scan(r.cnt, r.offs, E);
    if (lane == 0) p.offsets[E] = total;
  }
  __syncthreads();
  int mt = 0;
  for (int e = tid; e < E; e += kSkinnyThreads) {
    const int c = r.cnt[e];
    p.counts[e] = c;
    p.offsets[e] = r.offs[e];
    mt += (c + kSkinnyRows - 1) / kSkinnyRows;
  }
  atomicAdd(&r.mt, mt);
  // stable position: the group's offset plus the earlier slots of the same expert
  for (int s = tid; s < S; s += kSkinnyThreads) {
    const int e = r.ids[s];
    int rank = 0;
    for (int s2 = 0; s2 < s; ++s2) rank += r.ids[s2] == e ? 1 : 0;
    const int pos = r.offs[e] + rank;
    p.sorted_slot[pos] = s;
    p.slot_to_row[s] = pos;
  }
  // the routing went out by plain stores: write this XCD's L2 back before the flag
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    __hip_atomic_store(p.ctr + kCtrMtiles, y.xt + r.mt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.ctr + kCtrReady, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Gate/up tile (mtile, ntile); routed tiles first wait for the routing.
template <int BKG, int BKD>
__device__ __forceinline__ void gate_up_item(const FusedDecodeProblem& p, const Layout& y, FusedLds<BKG, BKD>& lds, int mtile,
                             int ntile) {
  int32_t* ctr = p.ctr;
  if (mtile >= y.xt) {
    wg_wait_ge(ctr + kCtrReady, 1, ctr + kCtrError);
    if (mtile >= load_agent(ctr + kCtrMtiles)) return;
  }
  if (skinny_tile<kNB, BKG, true, true>(p.gu, mtile, ntile, lds.g)) wg_signal(ctr + kCtrMtile0 + mtile);
}

// Down tile (mtile, ntile): waits for the routing (routed tiles) and its m-tile's gate/up tiles.
template <int BKG, int BKD>
__device__ __forceinline__ void down_item(const FusedDecodeProblem& p, const Layout& y, FusedLds<BKG, BKD>& lds, int mtile,
                          int ntile) {
  int32_t* ctr = p.ctr;
  if (mtile >= y.xt) {
    wg_wait_ge(ctr + kCtrReady, 1, ctr + kCtrError);
    if (mtile >= load_agent(ctr + kCtrMtiles)) return;
  }
  wg_wait_ge(ctr + kCtrMtile0 + mtile, y.nt_gu, ctr + kCtrError);
  if (skinny_tile<kNB, BKD, false, true>(p.dn, mtile, ntile, lds.d)) wg_signal(ctr + kCtrDnDone);
}

// Work item u = blockIdx.x.  Order: 0 publishes the routing; the shared expert's gate/up tiles; the
// routed gate/up tiles m-tile by m-tile, from the lag-th m-tile on each followed by the down tiles of
// the m-tile `lag` places earlier (so that a down tile usually finds its h complete); the remaining
// down tiles; the combine slices.  Every item waits only for items of smaller index.
template <int BKG, int BKD>
__global__ __launch_bounds__(kSkinnyThreads) void fused_decode_kernel(FusedDecodeProblem p, Layout y) {
  __shared__ FusedLds<BKG, BKD> lds;
  int u = blockIdx.x;
  if (u == 0) {
    const int E = p.E;
    if (E <= 64) publish_routing<1>(p, y, lds.r);
    else if (E <= 128) publish_routing<2>(p, y, lds.r);
    else if (E <= 192) publish_routing<3>(p, y, lds.r);
    else if (E <= 256) publish_routing<4>(p, y, lds.r);
    else publish_routing<5>(p, y, lds.r);   // E <= kFusedDecodeMaxExperts
    return;
  }
  u -= 1;
  if (u < y.xt * y.nt_gu) {
    gate_up_item(p, y, lds, u / y.nt_gu, u % y.nt_gu);
    return;
  }
  u -= y.xt * y.nt_gu;
  const int steps_a = min(y.lag, y.mt_r);
  if (u < steps_a * y.nt_gu) {
    gate_up_item(p, y, lds, y.xt + u / y.nt_gu, u % y.nt_gu);
    return;
  }
  u -= steps_a * y.nt_gu;
  const int steps_b = max(0, y.mt_r - y.lag);
  const int per_b = y.nt_gu + y.nt_dn;
  if (u < steps_b * per_b) {
    const int s = y.lag + u / per_b, r = u % per_b;
    if (r < y.nt_gu) gate_up_item(p, y, lds, y.xt + s, r);
    else down_item(p, y, lds, s - y.lag, r - y.nt_gu);
    return;
  }
  u -= steps_b * per_b;
  const int d0 = steps_b, n_c = y.xt + y.mt_r - steps_b;
  if (u < n_c * y.nt_dn) {
    down_item(p, y, lds, d0 + u / y.nt_dn, u % y.nt_dn);
    return;
  }
  u -= n_c * y.nt_dn;
  // combine: token u / ncpt, columns of slice u % ncpt, once every down tile is done
  int32_t* ctr = p.ctr;
  wg_wait_ge(ctr + kCtrReady, 1, ctr + kCtrError);
  const int n_mt = load_agent(ctr + kCtrMtiles);
  wg_wait_ge(ctr + kCtrDnDone, n_mt * y.nt_dn, ctr + kCtrError);
  const bool poison = load_agent(ctr + kCtrError) != 0;
  const int t = u / y.ncpt;
  const int h0 = (u - t * y.ncpt) * kCombineCols + (int)threadIdx.x * 8;
  if (t < p.T && h0 < p.H)
    combine_cols(p.dn.out, p.slot_to_row, p.w, p.dn.has_extra ? p.dn.out + (size_t)p.T * p.k * p.H : nullptr, t, h0,
                 p.k, p.H, p.out, poison);
}

Layout layout_of(const FusedDecodeProblem& p, int resident) {
  Layout y{};
  const int S = p.T * p.k;
  y.xt = p.gu.has_extra ? (p.T + kSkinnyRows - 1) / kSkinnyRows : 0;
  y.mt_r = std::min(p.E, S) + S / kSkinnyRows;   // every non-empty group adds at most one partial tile
  y.nt_gu = p.gu.N / skinny_bn<kNB, true>();
  y.nt_dn = p.dn.N / skinny_bn<kNB, false>();
  y.ncpt = (p.H + kCombineCols - 1) / kCombineCols;
  // about one GPU-full of gate/up items between a routed m-tile's gate/up and down items
  y.lag = std::max(1, (resident + y.nt_gu - 1) / y.nt_gu);
  return y;
}

// Workgroups of this kernel the GPU holds at once (compute units x resident workgroups per unit),
// looked up once per device and kernel instantiation.
constexpr int kMaxDevices = 64;
int g_resident[kMaxDevices][4];

template <int BKG, int BKD, int V>
moe_status_t launch_fused(const FusedDecodeProblem& p, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  int& resident = g_resident[dev][V];
  if (resident == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_decode_kernel<BKG, BKD>, kSkinnyThreads, 0) !=
            hipSuccess)
      return MOE_ERR_HIP;
    resident = std::max(1, cus * std::max(1, per_cu));
  }
  const Layout y = layout_of(p, resident);
  const long long items = 1 + (long long)(y.xt + y.mt_r) * (y.nt_gu + y.nt_dn) + (long long)p.T * y.ncpt;
  if (items > 0x7FFFFFFF) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL((fused_decode_kernel<BKG, BKD>), dim3((unsigned)items), dim3(kSkinnyThreads), 0, stream, p, y);
  return launch_status();
}

}  // namespace

int fused_decode_counter_words(int32_t T, int32_t k, int32_t E, bool shared) {
  const int S = T * k;
  return kCtrMtile0 + std::min(E, S) + S / kSkinnyRows + (shared ? (T + kSkinnyRows - 1) / kSkinnyRows : 0);
}

bool fused_decode_applies(const GemmProblem& gu, int32_t T, int32_t k) {
  if (T < 1 || T > kFusedDecodeMaxTokens || (int64_t)T * k > kFusedDecodeMaxSlots || k > kWave) return false;
  if (gu.bank.format != MOE_WEIGHT_NVFP4 || gu.G > kFusedDecodeMaxExperts) return false;
  if (gu.N % skinny_bn<kNB, true>() != 0 || gu.K % 128 != 0) return false;
  return grouped_gemm_uses_skinny_tiles(gu);
}

moe_status_t launch_fused_decode(const FusedDecodeProblem& p, hipStream_t stream) {
  if (!fused_decode_applies(p.gu, p.T, p.k)) return MOE_ERR_INVALID_ARGUMENT;
  if (p.dn.N % skinny_bn<kNB, false>() != 0 || p.dn.K % 128 != 0 || p.H % 8 != 0) return MOE_ERR_INVALID_ARGUMENT;
  const bool g256 = p.gu.K % 256 == 0, d256 = p.dn.K % 256 == 0;
  if (g256 && d256) return launch_fused<256, 256, 0>(p, stream);
  if (g256) return launch_fused<256, 128, 1>(p, stream);
  if (d256) return launch_fused<128, 256, 2>(p, stream);
  return launch_fused<128, 128, 3>(p, stream);
}

}  // namespace moe
