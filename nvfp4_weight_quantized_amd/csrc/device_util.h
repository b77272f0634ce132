// Device helpers shared by the route and permute kernels (header-only, inlined into each kernel).
// Wave-wide reductions and scans use DPP row operations and readlane (no LDS round trips).
#pragma once

#include "common.h"

namespace moe {

// v_mov_b32_dpp with the given control; lanes outside row_mask (or without a source) get `old`.
template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}

constexpr int kDppQuad1032 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuad2301 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
constexpr int kDppRowShr1 = 0x111;

// Monotone map of a float (not NaN) to uint32: a < b  <=>  key(a) < key(b); -0 and +0 share a key.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);   // -0 + 0 = +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Wave-wide max / min of uint32 returned to every lane (DPP row steps, then lane 63).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)dpp_i<kDppQuad1032>((int)x, (int)x));
  x = max(x, (uint32_t)dpp_i<kDppQuad2301>((int)x, (int)x));
  x = max(x, (uint32_t)dpp_i<kDppRowHalfMirror>((int)x, (int)x));
  x = max(x, (uint32_t)dpp_i<kDppRowMirror>((int)x, (int)x));
  x = max(x, (uint32_t)dpp_i<kDppRowBcast15, 0xA>((int)x, (int)x));
  x = max(x, (uint32_t)dpp_i<kDppRowBcast31, 0xC>((int)x, (int)x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, (uint32_t)dpp_i<kDppQuad1032>((int)x, (int)x));
  x = min(x, (uint32_t)dpp_i<kDppQuad2301>((int)x, (int)x));
  x = min(x, (uint32_t)dpp_i<kDppRowHalfMirror>((int)x, (int)x));
  x = min(x, (uint32_t)dpp_i<kDppRowMirror>((int)x, (int)x));
  x = min(x, (uint32_t)dpp_i<kDppRowBcast15, 0xA>((int)x, (int)x));
  x = min(x, (uint32_t)dpp_i<kDppRowBcast31, 0xC>((int)x, (int)x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Wave-wide sum returned to every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(dpp_i<kDppQuad1032>(__float_as_int(v), __float_as_int(v)));
  v += __int_as_float(dpp_i<kDppQuad2301>(__float_as_int(v), __float_as_int(v)));
  v += __int_as_float(dpp_i<kDppRowHalfMirror>(__float_as_int(v), __float_as_int(v)));
  v += __int_as_float(dpp_i<kDppRowMirror>(__float_as_int(v), __float_as_int(v)));
  v += __int_as_float(dpp_i<kDppRowBcast15, 0xA>(0, __float_as_int(v)));
  v += __int_as_float(dpp_i<kDppRowBcast31, 0xC>(0, __float_as_int(v)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Inclusive wave scan (lane order) of integers.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += dpp_i<kDppRowShr1, 0xF, true>(0, x);
  x += dpp_i<kDppRowShr1 + 1, 0xF, true>(0, x);   // row_shr:2
  x += dpp_i<kDppRowShr1 + 3, 0xF, true>(0, x);   // row_shr:4
  x += dpp_i<kDppRowShr1 + 7, 0xF, true>(0, x);   // row_shr:8
  x += dpp_i<kDppRowBcast15, 0xA>(0, x);
  x += dpp_i<kDppRowBcast31, 0xC>(0, x);
  return x;
}

// This lane's logits of one token (experts lane, lane + 64, ...), as topk_select takes them.
template <int VPL>
__device__ __forceinline__ void topk_load(const float* __restrict__ row, int E, float (&v)[VPL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < VPL; ++i) v[i] = row[min(lane + 64 * i, E - 1)];
}

// Top-k of one token's logits by one wavefront (E <= 64 * VPL, k <= 64), from the values topk_load
// gave this lane.  Returns, in lane j < k, the j-th selected expert and its renormalised softmax
// weight.  Equal logits -> lower index first; NaN ranks lowest.
// Lane l holds the logits of experts l, l + 64, ..., sorted descending (ties keep expert order);
// each of the k rounds takes the wave-wide maximum of the lanes' heads (as order keys) and, when
// several heads equal it, the lowest expert index among them; the winning lane (expert index
// mod 64) drops its head.
template <int VPL>
__device__ __forceinline__ void topk_select(const float (&raw)[VPL], int E, int k, int* out_id, float* out_w) {
  const int lane = threadIdx.x & 63;
  float v[VPL];
  int vi[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    const float val = raw[i];
    v[i] = (e < E && val == val) ? val : -INFINITY;
    vi[i] = e;
  }
  // insertion sort, descending; a later slot (higher expert index) moves up only if strictly larger
#pragma unroll
  for (int i = 1; i < VPL; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const bool swap = v[j] > v[j - 1];
      const float tv = v[j];
      const int ti = vi[j];
      v[j] = swap ? v[j - 1] : v[j];
      vi[j] = swap ? vi[j - 1] : vi[j];
      v[j - 1] = swap ? tv : v[j - 1];
      vi[j - 1] = swap ? ti : vi[j - 1];
    }
  float my_val = -INFINITY;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t key = order_key(v[0]);
    const uint32_t kmax = wave_max_u32(key);
    const uint64_t tied = __ballot(key == kmax);
    int bi;
    if (__popcll(tied) == 1)
      bi = __builtin_amdgcn_readlane(vi[0], __ffsll((unsigned long long)tied) - 1);
    else
      bi = (int)wave_min_u32(key == kmax ? (uint32_t)vi[0] : 0xFFFFFFFFu);
    const float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[0]), bi & 63));
    const bool win = (bi & 63) == lane;   // the winner drops its head
#pragma unroll
    for (int i = 0; i + 1 < VPL; ++i) {
      v[i] = win ? v[i + 1] : v[i];
      vi[i] = win ? vi[i + 1] : vi[i];
    }
    v[VPL - 1] = win ? -INFINITY : v[VPL - 1];
    vi[VPL - 1] = win ? 0x7FFFFFFF : vi[VPL - 1];
    my_val = (lane == j) ? bv : my_val;
    my_id = (lane == j) ? bi : my_id;
  }
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), 0));
  const float z = (lane < k) ? expf(my_val - top) : 0.f;
  const float s = wave_sum(z);
  *out_id = my_id;
  *out_w = z / s;
}

// Top-k of one token's logits row (topk_load, then topk_select).
template <int VPL>
__device__ __forceinline__ void topk_token(const float* __restrict__ row, int E, int k, int* out_id, float* out_w) {
  float raw[VPL];
  topk_load<VPL>(row, E, raw);
  topk_select<VPL>(raw, E, k, out_id, out_w);
}

// Calls f(IntC-like tag) with the smallest supported logits-per-lane count covering E (<= 1024).
template <int N>
struct Vpl {
  static constexpr int value = N;
};
template <typename F>
__device__ __forceinline__ void with_vpl(int E, F&& f) {
  if (E <= 64) f(Vpl<1>{});
  else if (E <= 128) f(Vpl<2>{});
  else if (E <= 192) f(Vpl<3>{});
  else if (E <= 256) f(Vpl<4>{});
  else if (E <= 320) f(Vpl<5>{});
  else if (E <= 384) f(Vpl<6>{});
  else if (E <= 512) f(Vpl<8>{});
  else f(Vpl<16>{});
}

// Exclusive scan of cnt[0..E) into out[0..E) by one wavefront (may be in place); returns the total.
__device__ __forceinline__ int wave_exclusive_scan(const int* cnt, int* out, int E) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    const int v = (e < E) ? cnt[e] : 0;
    const int incl = wave_inclusive_scan(v);
    if (e < E) out[e] = carry + incl - v;
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  return carry;
}

// Stable scatter of one wave's slots [s_begin, s_end): position = base[e] + rank among the earlier
// slots of the same expert in this wave's range; base[e] advances by the wave's count.  The lanes
// holding the same expert are found with one ballot per bit of the expert index (E <= 1024: at
// most 10), so no atomic ordering and no loop over distinct experts is involved.  A slot whose id
// lies outside [0, E) is placed nowhere: its slot_to_row entry is -1 (the histograms skip it too).
__device__ __forceinline__ void wave_stable_scatter(const int32_t* ids, int s_begin, int s_end, int E, int* base,
                                                    int32_t* __restrict__ sorted_slot,
                                                    int32_t* __restrict__ slot_to_row) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  const int nbits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;
  for (int s0 = s_begin; s0 < s_end; s0 += 64) {
    const int s = s0 + lane;
    const bool in_range = s < s_end;
    const int id = in_range ? ids[s] : 0;
    const bool valid = in_range && id >= 0 && id < E;
    const int e = valid ? id : 0;
    if (in_range && !valid) slot_to_row[s] = -1;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    if (valid) {
      const int rank = __popcll(peers & below);
      const int bb = base[e];
      const int pos = bb + rank;
      sorted_slot[pos] = s;
      slot_to_row[s] = pos;
      if (rank == 0) base[e] = bb + __popcll(peers);
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
  for (int s = s_begin + (tid & 63); s < s_end; s += 64) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&wave_hist[wave][e], 1);   // an id outside [0, E) joins no group
  }
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
  if (s_begin < s_end) wave_stable_scatter(ids, s_begin, s_end, E, wave_hist[wave], sorted_slot, slot_to_row);
}

}  // namespace moe
