// Device helpers shared by the route and permute kernels (header-only, inlined into each kernel).
#pragma once

#include "common.h"

namespace moe {

// Top-k of one token's logits by one wavefront (E <= 1024, k <= 64).  Returns, in lane j < k, the
// j-th selected expert and its renormalised softmax weight.  Equal logits -> lower index first;
// NaN ranks lowest.
__device__ __forceinline__ void topk_token(const float* __restrict__ row, int E, int k, int* out_id, float* out_w) {
  const int lane = threadIdx.x & 63;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    const float val = (e < E) ? row[e] : -INFINITY;
    v[i] = (val != val) ? -INFINITY : val;
  }
  uint32_t taken = 0;
#pragma unroll
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
  const float z = (lane < k) ? expf(my_val - top) : 0.f;
  float s = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  *out_id = my_id;
  *out_w = z / s;
}

// Exclusive scan of cnt[0..E) into out[0..E) by one wavefront (may be in place); returns the total.
__device__ __forceinline__ int wave_exclusive_scan(const int* cnt, int* out, int E) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    const int v = (e < E) ? cnt[e] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (e < E) out[e] = carry + incl - v;
    carry += __shfl(incl, 63);
  }
  return carry;
}

// Stable scatter of one wave's slots [s_begin, s_end): position = base[e] + rank among the earlier
// slots of the same expert in this wave's range; base[e] advances by the wave's count.  Ranks
// come from ballots over the lanes holding the same expert, so no atomic ordering is involved.
__device__ __forceinline__ void wave_stable_scatter(const int32_t* ids, int s_begin, int s_end, int* base,
                                                    int32_t* __restrict__ sorted_slot,
                                                    int32_t* __restrict__ slot_to_row) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int s0 = s_begin; s0 < s_end; s0 += 64) {
    const int s = s0 + lane;
    const bool valid = s < s_end;
    const int e = valid ? ids[s] : -1;
    uint64_t rem = __ballot(valid);
    uint64_t peers = 0;
    while (rem) {
      const int leader = __ffsll((unsigned long long)rem) - 1;
      const int le = __shfl(e, leader);
      const uint64_t m = __ballot(valid && e == le);
      if (valid && e == le) peers = m;
      rem &= ~m;
    }
    if (valid) {
      const int rank = __popcll(peers & below);
      const int b = base[e];
      const int pos = b + rank;
      sorted_slot[pos] = s;
      slot_to_row[s] = pos;
      if (rank == 0) base[e] = b + __popcll(peers);
    }
  }
}

constexpr int kPermWaves = kPermuteThreads / kWave;           // 8
constexpr int kPermSlotsPerWave = kPermuteChunk / kPermWaves; // 256
constexpr int kPermMaxE = 1024;

// Whole permutation of S <= kPermuteChunk slots by one workgroup of kPermuteThreads threads.
// `ids` may live in LDS or global memory.  wave_hist: [kPermWaves][kPermMaxE], offs: [kPermMaxE] (LDS).
__device__ __forceinline__ void permute_block(const int32_t* ids, int S, int E, int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
                                              int32_t* __restrict__ slot_to_row, int (*wave_hist)[kPermMaxE],
                                              int* offs) {
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int w = 0; w < kPermWaves; ++w)
    for (int e = tid; e < E; e += kPermuteThreads) wave_hist[w][e] = 0;
  __syncthreads();
  const int s_begin = wave * kPermSlotsPerWave;
  const int s_end = min(S, s_begin + kPermSlotsPerWave);
  for (int s = s_begin + (tid & 63); s < s_end; s += 64) atomicAdd(&wave_hist[wave][ids[s]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += kPermuteThreads) {
    int c = 0;
    for (int w = 0; w < kPermWaves; ++w) c += wave_hist[w][e];
    counts[e] = c;
    offs[e] = c;
  }
  __syncthreads();
  if (wave == 0) {
    const int total = wave_exclusive_scan(offs, offs, E);
    if ((tid & 63) == 0) offsets[E] = total;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermuteThreads) {
    offsets[e] = offs[e];
    int run = offs[e];
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = wave_hist[w][e];
      wave_hist[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  if (s_begin < s_end) wave_stable_scatter(ids, s_begin, s_end, wave_hist[wave], sorted_slot, slot_to_row);
}

}  // namespace moe
