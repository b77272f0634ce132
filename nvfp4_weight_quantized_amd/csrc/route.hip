// Router (S1) and top-k selection (S2) of the NVFP4 MoE layer, gfx950.
//
// S1: logits[t][e] = sum_h x[t][h] * Wr[e][h] (+ bias[e]), bf16 inputs, fp32 accumulation.
//     Few tokens: one workgroup per (expert, 8 tokens) streams the expert's router row once with
//     every load of a pass in flight together (the router weight is the only real traffic).  Many
//     tokens: an LDS-tiled bf16 MFMA GEMM (16x16x32 fragments).
// S2: one wavefront per token: each lane sorts its few logits, then k rounds of a wave-wide
//     argmax over the lanes' heads (equal logits -> lower index), then the softmax over the k
//     selected logits (equal to the full softmax renormalised over the selection).
// Sources: router -> top-k stage of the modular fused MoE ("vLLM on the NVIDIA DGX Spark: A
// Complete Technical Guide", section 7.1); top-8 of 320 routed experts ("Serving Solar Open 2 on
// DGX Spark", "Solar Open 2 in brief").
#include "device_util.h"

namespace moe {
namespace {

constexpr int kGemvMaxTokens = 32;
constexpr int kGemvTokens = 8;     // tokens per workgroup

// Few tokens: one workgroup per (expert, group of up to 8 tokens).  Each thread takes 8
// consecutive h of the expert's router row per 2048-wide pass and dots them with the same h of
// every token, all loads of a pass issued together; the per-token sums are then reduced across
// the workgroup (wave sums, then the four waves in order).
__global__ __launch_bounds__(256) void router_small_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr,
                                                           const float* __restrict__ bias, int T, int H, int E,
                                                           float* __restrict__ logits) {
  __shared__ float part[4][kGemvTokens];
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

// C[T][E] = X[T][H] . Wr[E][H]^T with bf16 MFMA; 64x64 tile per workgroup, 4 waves of 32x32.
constexpr int kRB = 64;       // tile rows / cols
constexpr int kRK = 64;       // K chunk
constexpr int kRPad = 8;      // bf16 padding per LDS row (16 bytes) against bank conflicts

__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          const float* __restrict__ bias, int T, int H,
                                                          int E, float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kRB][kRK + kRPad];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kRB][kRK + kRPad];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int row0 = blockIdx.y * kRB;
  const int col0 = blockIdx.x * kRB;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // each thread moves 2 x 16 bytes of A and of B per chunk: row = tid/8 (+32), col8 = tid%8
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  for (int k0 = 0; k0 < H; k0 += kRK) {
    uint4 av[2], bv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = lr + 32 * i;
      av[i] = (row0 + r < T) ? *reinterpret_cast<const uint4*>(x + (size_t)(row0 + r) * H + k0 + lc)
                             : uint4{0, 0, 0, 0};
      bv[i] = (col0 + r < E) ? *reinterpret_cast<const uint4*>(wr + (size_t)(col0 + r) * H + k0 + lc)
                             : uint4{0, 0, 0, 0};
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<uint4*>(&As[lr + 32 * i][lc]) = av[i];
      *reinterpret_cast<uint4*>(&Bs[lr + 32 * i][lc]) = bv[i];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kRK; kk += 32) {
      bf16x8 af[2], bfr[2];
      const int q = lane >> 4, m = lane & 15;
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
  const int q = lane >> 4, n = lane & 15;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = col0 + wn * 32 + j * 16 + n;
    if (col >= E) continue;
    const float b = bias ? bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + wm * 32 + i * 16 + 4 * q + r;
        if (row < T) logits[(size_t)row * E + col] = acc[i][j][r] + b;
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

}  // namespace

moe_status_t launch_router_logits(const uint16_t* x, const uint16_t* w_router, const float* bias, int32_t T,
                                  int32_t H, int32_t E, float* logits, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  if (T <= kGemvMaxTokens) {
    hipLaunchKernelGGL(router_small_kernel, dim3(E, (T + kGemvTokens - 1) / kGemvTokens), dim3(256), 0, stream, x,
                       w_router, bias, (int)T, (int)H, (int)E, logits);
  } else {
    hipLaunchKernelGGL(router_mfma_kernel, dim3((E + kRB - 1) / kRB, (T + kRB - 1) / kRB), dim3(256), 0, stream, x,
                       w_router, bias, (int)T, (int)H, (int)E, logits);
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
