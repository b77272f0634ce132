// Router (S1) and top-k selection (S2) of the NVFP4 MoE layer, gfx950.
//
// S1: logits[t][e] = sum_h x[t][h] * Wr[e][h] (+ bias[e]), bf16 inputs, fp32 accumulation.
//     Few tokens: one workgroup per (expert, 8 tokens) streams the expert's router row once with
//     every load of a pass in flight together (the router weight is the only real traffic).  Many
//     tokens: a bf16 MFMA GEMM (16x16x32 fragments) on LDS-staged 64x64 tiles.
// S2: one wavefront per token: each lane sorts its few logits, then k rounds of a wave-wide
//     argmax over the lanes' heads (equal logits -> lower index), then the softmax over the k
//     selected logits (equal to the full softmax renormalised over the selection).
// Sources: router -> top-k stage of the modular fused MoE ("vLLM on the NVIDIA DGX Spark: A
// Complete Technical Guide", section 7.1); top-8 of 320 routed experts ("Serving Solar Open 2 on
// DGX Spark", "Solar Open 2 in brief").
#include "device_util.h"

namespace moe {
namespace {

constexpr int kGemvMaxTokens = kRouterSmallTokens;
constexpr int kGemvTokens = 8;     // tokens per workgroup

// Few tokens: one workgroup per (expert, group of up to 8 tokens).  Each thread takes 8
// consecutive h of the expert's router row per 2048-wide pass and dots them with the same h of
// every token, all loads of a pass issued together; the per-token sums are then reduced across
// the workgroup (wave sums, then the four waves in order).
// `zero` (optional): n_zero words the first workgroup clears (counters of the kernels that follow
// in the same stream: the fused decode kernel's hand-offs, the grouped GEMMs' tile counters).
__global__ __launch_bounds__(256) void router_small_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr,
                                                           const float* __restrict__ bias, int T, int H, int E,
                                                           float* __restrict__ logits, int32_t* __restrict__ zero,
                                                           int n_zero) {
  __shared__ float part[4][kGemvTokens];
  if (zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < n_zero; i += 256) zero[i] = 0;
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * kGemvTokens;
  const int tn = min(kGemvTokens, T - t0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* wrow = wr + (size_t)e * H;
  float acc[kGemvTokens];
#pragma unroll
  for (int t = 0; t < kGemvTokens; ++t) acc[t] = 0.f;
#pragma unroll 2
  for (int h0 = threadIdx.x * 8; h0 < H; h0 += 256 * 8) {
    const uint4 wv = *reinterpret_cast<const uint4*>(wrow + h0);
    uint4 xv[kGemvTokens];
#pragma unroll
    for (int t = 0; t < kGemvTokens; ++t)
      xv[t] = *reinterpret_cast<const uint4*>(x + (size_t)(t0 + min(t, tn - 1)) * H + h0);
    const uint32_t wq[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int t = 0; t < kGemvTokens; ++t) {
      const uint32_t xq[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[t] = fmaf(__uint_as_float(xq[i] << 16), __uint_as_float(wq[i] << 16), acc[t]);
        acc[t] = fmaf(__uint_as_float(xq[i] & 0xFFFF0000u), __uint_as_float(wq[i] & 0xFFFF0000u), acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kGemvTokens; ++t) {
    const float v = wave_sum(acc[t]);
    if (lane == 0) part[wave][t] = v;
  }
  __syncthreads();
  if (threadIdx.x < tn) {
    const int t = threadIdx.x;
    const float v = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
    logits[(size_t)(t0 + t) * E + e] = v + (bias ? bias[e] : 0.f);
  }
}

// C[T][E] = X[T][H] . Wr[E][H]^T with bf16 MFMA (16x16x32), fp32 accumulation; 64 tokens x 64
// experts per workgroup, 4 waves of 32x32, K chunks of 128 staged in LDS.  Each chunk is loaded
// into registers while the previous one is multiplied (one chunk in flight), then written to LDS
// between two barriers.  Tiles are numbered so that the expert blocks of one token block run on one
// XCD (workgroup b runs on XCD b % 8) and read its x rows from that XCD's L2.
// splits > 1: the K range of each tile is cut into `splits` contiguous runs of chunks, one per
// workgroup; run s writes its partial sums, without the bias, to logits (s = 0) or to
// partial[s - 1] ([T][E] each), and topk_sum_kernel adds them.  The chunks of a workgroup run one
// after another at the latency of a load each, so fewer of them per workgroup (and more workgroups
// when the tiles alone leave compute units idle) shorten the launch.
constexpr int kRB = 64;                    // tile rows (tokens) and columns (experts)
constexpr int kRK = 128;                   // K chunk
constexpr int kRPad = 8;                   // bf16 of padding per LDS row (16 bytes)
constexpr int kRTpr = kRK / 8;             // threads per tile row per chunk (16 bytes each)
constexpr int kRRpp = 256 / kRTpr;         // tile rows per pass
constexpr int kRIt = kRB / kRRpp;          // passes
constexpr int kRXcds = 8;
constexpr int kRouterMaxSplits = 4;        // K splits of the router GEMM (router_k_splits)
typedef uint32_t u32x4_r __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          const float* __restrict__ bias, int T, int H,
                                                          int E, float* __restrict__ logits,
                                                          int32_t* __restrict__ zero, int n_zero,
                                                          float* __restrict__ partial, int splits) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kRB][kRK + kRPad];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kRB][kRK + kRPad];
  const int tid = threadIdx.x;
  if (zero && blockIdx.x == 0)
    for (int i = tid; i < n_zero; i += 256) zero[i] = 0;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int eb = (E + kRB - 1) / kRB;
  const int total = eb * ((T + kRB - 1) / kRB) * splits;
  const int per_xcd = (total + kRXcds - 1) / kRXcds;
  const int L = (blockIdx.x % kRXcds) * per_xcd + blockIdx.x / kRXcds;
  if (L >= total) return;
  const int tile = L / splits, split = L % splits;
  const int row0 = (tile / eb) * kRB;
  const int col0 = (tile % eb) * kRB;
  const int nKall = H / kRK;
  const int c0 = split * nKall / splits, c1 = (split + 1) * nKall / splits;

  // this thread copies 16 bytes at column lc of tile rows lr + kRRpp*i (rows past T or E repeat
  // the last valid row; their results are not stored)
  const int lr = tid / kRTpr, lc = (tid % kRTpr) * 8;
  const uint16_t* xrow[kRIt];
  const uint16_t* wrow[kRIt];
#pragma unroll
  for (int i = 0; i < kRIt; ++i) {
    xrow[i] = x + (size_t)min(row0 + lr + kRRpp * i, T - 1) * H + lc;
    wrow[i] = wr + (size_t)min(col0 + lr + kRRpp * i, E - 1) * H + lc;
  }
  u32x4_r av[kRIt], bv[kRIt];
#pragma unroll
  for (int i = 0; i < kRIt; ++i) {
    av[i] = *reinterpret_cast<const u32x4_r*>(xrow[i] + (size_t)c0 * kRK);
    bv[i] = *reinterpret_cast<const u32x4_r*>(wrow[i] + (size_t)c0 * kRK);
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int q = lane >> 4, m = lane & 15;
  for (int c = c0; c < c1; ++c) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRIt; ++i) {
      *reinterpret_cast<u32x4_r*>(&As[lr + kRRpp * i][lc]) = av[i];
      *reinterpret_cast<u32x4_r*>(&Bs[lr + kRRpp * i][lc]) = bv[i];
    }
    __syncthreads();
    if (c + 1 < c1) {
#pragma unroll
      for (int i = 0; i < kRIt; ++i) {
        av[i] = *reinterpret_cast<const u32x4_r*>(xrow[i] + (size_t)(c + 1) * kRK);
        bv[i] = *reinterpret_cast<const u32x4_r*>(wrow[i] + (size_t)(c + 1) * kRK);
      }
    }
#pragma unroll
    for (int kk = 0; kk < kRK; kk += 32) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(&As[wm * 32 + i * 16 + m][kk + 8 * q]);
        bfr[i] = *reinterpret_cast<const bf16x8*>(&Bs[wn * 32 + i * 16 + m][kk + 8 * q]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  // lane (q, n) of block (i, j): tokens 4q + r, expert n
  float* out = split == 0 ? logits : partial + (size_t)(split - 1) * T * E;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = col0 + wn * 32 + j * 16 + m;
    if (col >= E) continue;
    const float b = (bias && splits == 1) ? bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + wm * 32 + i * 16 + 4 * q + r;
        if (row < T) out[(size_t)row * E + col] = acc[i][j][r] + b;
      }
  }
}

// One wave per token.  E <= 1024 (16 logits per lane), k <= 64.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int id;
  float wt;
  with_vpl(E, [&](auto vpl) { topk_token<decltype(vpl)::value>(logits + (size_t)t * E, E, k, &id, &wt); });
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    w[(size_t)t * k + lane] = wt;
  }
}

// One wave per token, after the split router: the token's logits are the partial sums added in
// split order, then the bias (written back to `logits`), and then its top-k as topk_kernel.
__global__ __launch_bounds__(256) void topk_sum_kernel(float* __restrict__ logits, const float* __restrict__ partial,
                                                       int splits, const float* __restrict__ bias, int T, int E,
                                                       int k, int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int id;
  float wt;
  with_vpl(E, [&](auto vpl) {
    constexpr int VPL = decltype(vpl)::value;
    // every load of the token issued together (at most kRouterMaxSplits parts), then the sums in
    // split order
    float part[VPL][kRouterMaxSplits];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const size_t at = (size_t)t * E + min(lane + 64 * i, E - 1);
      part[i][0] = logits[at];
#pragma unroll
      for (int s = 1; s < kRouterMaxSplits; ++s) part[i][s] = s < splits ? partial[(size_t)(s - 1) * T * E + at] : 0.f;
    }
    float raw[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      float v = part[i][0];
#pragma unroll
      for (int s = 1; s < kRouterMaxSplits; ++s)
        if (s < splits) v += part[i][s];
      if (bias) v += bias[min(e, E - 1)];
      raw[i] = v;
      if (e < E) logits[(size_t)t * E + e] = v;
    }
    topk_select<VPL>(raw, E, k, &id, &wt);
  });
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    w[(size_t)t * k + lane] = wt;
  }
}

}  // namespace

int router_k_splits(int32_t T, int32_t H, int32_t E, int32_t k) {
  if (T <= kGemvMaxTokens || (int64_t)T * k <= kPermuteChunk || H < 2 * kRK) return 1;
  const long long tiles = (long long)((E + kRB - 1) / kRB) * ((T + kRB - 1) / kRB);
  const int s = tiles >= 1024 ? 1 : tiles >= 256 ? 2 : 4;
  return std::min(s, H / kRK);
}

moe_status_t launch_topk_sum(float* logits, const float* partial, int32_t splits, const float* bias, int32_t T,
                             int32_t E, int32_t k, int32_t* ids, float* w, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  if (splits < 1 || splits > kRouterMaxSplits || (splits > 1 && !partial)) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(topk_sum_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits, partial, (int)splits, bias,
                     (int)T, (int)E, (int)k, ids, w);
  return launch_status();
}

moe_status_t launch_router_logits(const uint16_t* x, const uint16_t* w_router, const float* bias, int32_t T,
                                  int32_t H, int32_t E, float* logits, hipStream_t stream, int32_t* zero,
                                  int32_t n_zero, float* partial, int32_t splits) {
  if (T == 0) return MOE_OK;
  if (T <= kGemvMaxTokens) {
    hipLaunchKernelGGL(router_small_kernel, dim3(E, (T + kGemvTokens - 1) / kGemvTokens), dim3(256), 0, stream, x,
                       w_router, bias, (int)T, (int)H, (int)E, logits, zero, (int)n_zero);
  } else {
    if (H % kRK != 0 || splits < 1 || splits > H / kRK || (splits > 1 && !partial)) return MOE_ERR_INVALID_ARGUMENT;
    const long long tiles = (long long)((E + kRB - 1) / kRB) * ((T + kRB - 1) / kRB) * splits;
    const long long grid = (tiles + kRXcds - 1) / kRXcds * kRXcds;
    if (grid > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(router_mfma_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, w_router, bias, (int)T,
                       (int)H, (int)E, logits, zero, (int)n_zero, partial, (int)splits);
  }
  return launch_status();
}

moe_status_t launch_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int32_t T,
                          int32_t H, int32_t E, int32_t k, bool logits_given, float* logits,
                          int32_t* ids, float* w, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  if (!logits_given) {
    if (moe_status_t st = launch_router_logits(x, w_router, bias, T, H, E, logits, stream)) return st;
  }
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits, (int)T, (int)E, (int)k, ids, w);
  return launch_status();
}

}  // namespace moe
