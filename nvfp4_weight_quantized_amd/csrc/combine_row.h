// The combine (S6) of one token over one slice of its columns, shared by the stand-alone combine
// kernel and the fused decode kernel: the top-k-weighted reduction of the expert rows of the token
// plus the shared expert's row ("vLLM on the NVIDIA DGX Spark: A Complete Technical Guide",
// section 4: fused MoE with top-k-weight reduction; "Serving Solar Open 2 on DGX Spark": one shared
// expert used by every token, added here with weight 1).
//
// out[t][h] = bf16( sum_{j<k} w[t][j] * y[slot_to_row[t*k+j]][h]  +  y_shared[t][h] ),
// accumulated in fp32 in that order.  A gather-add: each thread owns 8 consecutive columns and
// reads 16-byte pieces of the k+1 source rows; no atomics, so the result is deterministic.
// A negative row (a slot the permutation placed nowhere because its expert id was out of range)
// is never read: the token's output row becomes NaN instead, a loud result.
#pragma once

#include "common.h"

namespace moe {
namespace {

constexpr int kCombineThreads = 256;
constexpr int kCombineCols = kCombineThreads * 8;  // columns per workgroup
typedef uint32_t u32x4_c __attribute__((ext_vector_type(4)));

// Columns [h0, h0 + 8) of token t (one thread); `poison` writes NaN instead.
__device__ __forceinline__ void combine_cols(const uint16_t* __restrict__ y, const int32_t* __restrict__ slot_to_row,
                                             const float* __restrict__ w, const uint16_t* __restrict__ y_shared,
                                             int t, int h0, int k, int H, uint16_t* __restrict__ out, bool poison) {
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  // the k source rows in groups of 8: indices and weights first, then all row loads, then the
  // fma chain in j order (every load of a group in flight together)
  bool placed = !poison;
  for (int j0 = 0; j0 < k; j0 += 8) {
    int rows[8];
    float wj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + u, k - 1);
      const int r = slot_to_row[(size_t)t * k + j];
      placed = placed && r >= 0;
      rows[u] = max(r, 0);
      wj[u] = w[(size_t)t * k + j];
    }
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // each expert row is read once: stream it past the caches
      const u32x4_c q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_c*>(y + (size_t)rows[u] * H + h0));
      v[u] = uint4{q[0], q[1], q[2], q[3]};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < k) {
        const uint32_t q[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(wj[u], __uint_as_float(q[i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(wj[u], __uint_as_float(q[i] & 0xFFFF0000u), acc[2 * i + 1]);
        }
      }
    }
  }
  if (y_shared) {
    const uint4 v = *reinterpret_cast<const uint4*>(y_shared + (size_t)t * H + h0);
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(q[i] << 16);
      acc[2 * i + 1] += __uint_as_float(q[i] & 0xFFFF0000u);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = placed ? f32x2_to_bf16x2(acc[2 * i], acc[2 * i + 1]) : 0x7FC07FC0u;   // two bf16 quiet NaNs
  *reinterpret_cast<uint4*>(out + (size_t)t * H + h0) = uint4{o[0], o[1], o[2], o[3]};
}

}  // namespace
}  // namespace moe
