// Router (S1) and top-k selection (S2) of the NVFP4 MoE layer, gfx950.
//
// S1: logits[t][e] = sum_h x[t][h] * Wr[e][h] (+ bias[e]), bf16 inputs, fp32 accumulation.
//     Few tokens: one wavefront per expert streams its router row once and dots it with every
//     token (the router weight is the only real traffic).  Many tokens: an LDS-tiled bf16 MFMA
//     GEMM (16x16x32 fragments).
// S2: one wavefront per token: k rounds of a wave-wide argmax (equal logits -> lower index),
//     then the softmax over the k selected logits (equal to the full softmax renormalised over
//     the selection).
// Sources: router -> top-k stage of the modular fused MoE ("vLLM on the NVIDIA DGX Spark: A
// Complete Technical Guide", section 7.1); top-8 of 320 routed experts ("Serving Solar Open 2 on
// DGX Spark", "Solar Open 2 in brief").
#include "common.h"

namespace moe {
namespace {

constexpr int kGemvMaxTokens = 32;

// One wave per expert; 4 waves per workgroup.
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          const float* __restrict__ bias, int T, int H,
                                                          int E, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  float acc[kGemvMaxTokens];
#pragma unroll
  for (int t = 0; t < kGemvMaxTokens; ++t) acc[t] = 0.f;
  const uint16_t* wrow = wr + (size_t)e * H;
  for (int h0 = lane * 8; h0 < H; h0 += 512) {
    const uint4 wv = *reinterpret_cast<const uint4*>(wrow + h0);
    const uint32_t wq[4] = {wv.x, wv.y, wv.z, wv.w};
    float wf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wf[2 * i] = __uint_as_float(wq[i] << 16);
      wf[2 * i + 1] = __uint_as_float(wq[i] & 0xFFFF0000u);
    }
#pragma unroll
    for (int t = 0; t < kGemvMaxTokens; ++t) {
      if (t < T) {
        const uint4 xv = *reinterpret_cast<const uint4*>(x + (size_t)t * H + h0);
        const uint32_t xq[4] = {xv.x, xv.y, xv.z, xv.w};
        float s = acc[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s = fmaf(__uint_as_float(xq[i] << 16), wf[2 * i], s);
          s = fmaf(__uint_as_float(xq[i] & 0xFFFF0000u), wf[2 * i + 1], s);
        }
        acc[t] = s;
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int t = 0; t < kGemvMaxTokens; ++t) {
    if (t < T) {
      float v = acc[t];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0) logits[(size_t)t * E + e] = v + b;
    }
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
  const float* row = logits + (size_t)t * E;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    float val = (e < E) ? row[e] : -INFINITY;
    v[i] = (val != val) ? -INFINITY : val;  // NaN ranks lowest
  }
  uint32_t taken = 0;
  for (int i = 0; i < 16; ++i)
    if (lane + 64 * i >= E) taken |= 1u << i;
  float my_val = -INFINITY;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + 64 * i;
      if (!((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) {
      my_val = bv;
      my_id = bi;
    }
  }
  const float top = __shfl(my_val, 0);
  float z = (lane < k) ? expf(my_val - top) : 0.f;
  float s = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = z / s;
  }
}

}  // namespace

moe_status_t launch_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int32_t T,
                          int32_t H, int32_t E, int32_t k, bool logits_given, float* logits,
                          int32_t* ids, float* w, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  if (!logits_given) {
    if (T <= kGemvMaxTokens) {
      hipLaunchKernelGGL(router_gemv_kernel, dim3((E + 3) / 4), dim3(256), 0, stream, x, w_router, bias,
                         (int)T, (int)H, (int)E, logits);
    } else {
      hipLaunchKernelGGL(router_mfma_kernel, dim3((E + kRB - 1) / kRB, (T + kRB - 1) / kRB), dim3(256), 0,
                         stream, x, w_router, bias, (int)T, (int)H, (int)E, logits);
    }
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  }
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits, (int)T, (int)E, (int)k,
                     ids, w);
  return launch_status();
}

}  // namespace moe
