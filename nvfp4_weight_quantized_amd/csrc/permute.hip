// Token permutation (S3) of the NVFP4 MoE layer, gfx950.
//
// Groups the S = T*k slots (slot = t*k + j) by expert, keeping slot order inside each group, and
// writes per-expert counts, exclusive offsets, the sorted slot list and its inverse.  The result
// is bit-exact and independent of scheduling: counts come from LDS integer atomics (order-free),
// and every slot's position is its group offset plus the number of earlier slots of the same
// expert, computed from per-block and per-wave histograms and in-wave ballots -- never from the
// order in which atomics land; lanes of one wave holding the same expert are found with ballots.
//
// Small S (one workgroup): one launch does histogram, scan and scatter; for few tokens the top-k
// selection (S2) runs in the same launch.  Larger S: per-block histograms, then per-block stable
// scatter, each scatter workgroup scanning the histograms itself (up to 16 blocks) or after one
// scan workgroup (more blocks).
// Source: the "Permute-Experts-Unpermute" stage of the modular fused MoE ("vLLM on the NVIDIA DGX
// Spark: A Complete Technical Guide", section 7.1) and the token dispatch of the fused b12x MoE
// (section 4).
#include "device_util.h"

namespace moe {
namespace {

// One workgroup does everything (S <= kPermuteChunk).
__global__ __launch_bounds__(kPermuteThreads) void permute_single_kernel(
    const int32_t* __restrict__ ids, int S, int E, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_to_row) {
  __shared__ int wave_hist[kPermWaves][kPermMaxE];
  __shared__ int offs[kPermMaxE];
  permute_block(ids, S, E, counts, offsets, sorted_slot, slot_to_row, wave_hist, offs);
}

// S2 + S3 for few tokens in one workgroup: each wave selects the top-k of its tokens, then the
// block permutes the selection from LDS.
__global__ __launch_bounds__(kPermuteThreads) void topk_permute_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ slot_to_row) {
  __shared__ int wave_hist[kPermWaves][kPermMaxE];
  __shared__ int offs[kPermMaxE];
  __shared__ int ids_s[kPermuteChunk];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t = wave; t < T; t += kPermWaves) {
    int id;
    float wt;
    with_vpl(E, [&](auto vpl) { topk_token<decltype(vpl)::value>(logits + (size_t)t * E, E, k, &id, &wt); });
    if (lane < k) {
      ids[(size_t)t * k + lane] = id;
      w[(size_t)t * k + lane] = wt;
      ids_s[t * k + lane] = id;
    }
  }
  __syncthreads();
  permute_block(ids_s, T * k, E, counts, offsets, sorted_slot, slot_to_row, wave_hist, offs);
}

// Multi-block path, step 1: per-block histograms block_hist[b][e].
__global__ __launch_bounds__(kPermuteThreads) void permute_hist_kernel(const int32_t* __restrict__ ids, int S,
                                                                       int E, int32_t* __restrict__ block_hist) {
  __shared__ int hist[kPermMaxE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPermuteThreads) hist[e] = 0;
  __syncthreads();
  const int s_begin = blockIdx.x * kPermuteChunk;
  const int s_end = min(S, s_begin + kPermuteChunk);
  for (int s = s_begin + tid; s < s_end; s += kPermuteThreads) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);   // an id outside [0, E) joins no group
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermuteThreads) block_hist[(size_t)blockIdx.x * E + e] = hist[e];
}

// Step 2 (one workgroup): counts, offsets, and block_hist[b][e] -> first row of block b in group e.
// Each thread owns experts e; the per-block counts of e are read kScanBatch at a time, all loads of
// a batch in flight together (in one loop of dependent read-then-write the loads would wait for
// the stores before them, which may alias).
constexpr int kScanBatch = 16;
__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* __restrict__ block_hist, int nb, int E,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int offs[kPermMaxE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int b0 = 0; b0 < nb; b0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) v[i] = (b0 + i < nb) ? block_hist[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) run += v[i];
    }
    counts[e] = run;
    offs[e] = run;
  }
  __syncthreads();
  if (tid < 64) {
    const int total = wave_exclusive_scan(offs, offs, E);
    if (tid == 0) offsets[E] = total;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    offsets[e] = offs[e];
    int run = offs[e];
    for (int b0 = 0; b0 < nb; b0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) v[i] = (b0 + i < nb) ? block_hist[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) {
        if (b0 + i < nb) block_hist[(size_t)(b0 + i) * E + e] = run;
        run += v[i];
      }
    }
  }
}

// Step 3: per-block stable scatter from the block bases.
__global__ __launch_bounds__(kPermuteThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int S, int E, const int32_t* __restrict__ block_base,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_to_row) {
  __shared__ int wave_hist[kPermWaves][kPermMaxE];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int w = 0; w < kPermWaves; ++w)
    for (int e = tid; e < E; e += kPermuteThreads) wave_hist[w][e] = 0;
  __syncthreads();
  const int blk0 = blockIdx.x * kPermuteChunk;
  const int s_begin = blk0 + wave * kPermSlotsPerWave;
  const int s_end = min(S, s_begin + kPermSlotsPerWave);
  for (int s = s_begin + (tid & 63); s < s_end; s += 64) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&wave_hist[wave][e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermuteThreads) {
    int run = block_base[(size_t)blockIdx.x * E + e];
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = wave_hist[w][e];
      wave_hist[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  if (s_begin < s_end) wave_stable_scatter(ids, s_begin, s_end, E, wave_hist[wave], sorted_slot, slot_to_row);
}

// Steps 2 and 3 in one launch for up to kScanInScatter blocks: every scatter workgroup reads all
// the per-block histograms (nb * E values, from L2), forms the counts, their exclusive scan and its
// own block's bases, then scatters as above; workgroup 0 writes counts and offsets.  One launch
// fewer than scan then scatter, for S <= kScanInScatter * kPermuteChunk.
constexpr int kScanInScatter = 16;
__global__ __launch_bounds__(kPermuteThreads) void permute_scan_scatter_kernel(
    const int32_t* __restrict__ ids, int S, int E, int nb, const int32_t* __restrict__ block_hist,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ slot_to_row) {
  __shared__ int wave_hist[kPermWaves][kPermMaxE];
  __shared__ int offs[kPermMaxE];
  __shared__ int before[kPermMaxE];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int b = blockIdx.x;
  // per expert: the count over all blocks and the part of it in the blocks before this one
  for (int e = tid; e < E; e += kPermuteThreads) {
    int v[kScanInScatter];
#pragma unroll
    for (int i = 0; i < kScanInScatter; ++i) v[i] = i < nb ? block_hist[(size_t)i * E + e] : 0;
    int total = 0, pre = 0;
#pragma unroll
    for (int i = 0; i < kScanInScatter; ++i) {
      pre = i == b ? total : pre;
      total += v[i];
    }
    offs[e] = total;
    before[e] = pre;
    if (b == 0) counts[e] = total;
  }
  for (int w = 0; w < kPermWaves; ++w)
    for (int e = tid; e < E; e += kPermuteThreads) wave_hist[w][e] = 0;
  __syncthreads();
  const int blk0 = b * kPermuteChunk;
  const int s_begin = blk0 + wave * kPermSlotsPerWave;
  const int s_end = min(S, s_begin + kPermSlotsPerWave);
  if (wave == 0) {
    const int total = wave_exclusive_scan(offs, offs, E);
    if (b == 0 && (tid & 63) == 0) offsets[E] = total;
  }
  for (int s = s_begin + (tid & 63); s < s_end; s += 64) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&wave_hist[wave][e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermuteThreads) {
    if (b == 0) offsets[e] = offs[e];
    int run = offs[e] + before[e];
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = wave_hist[w][e];
      wave_hist[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  if (s_begin < s_end) wave_stable_scatter(ids, s_begin, s_end, E, wave_hist[wave], sorted_slot, slot_to_row);
}

}  // namespace

moe_status_t launch_permute(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
                            int32_t* offsets, int32_t* sorted_slot, int32_t* slot_to_row,
                            int32_t* block_hist, hipStream_t stream) {
  const int S = T * k;
  if (S <= kPermuteChunk) {
    hipLaunchKernelGGL(permute_single_kernel, dim3(1), dim3(kPermuteThreads), 0, stream, ids, S, (int)E, counts,
                       offsets, sorted_slot, slot_to_row);
    return launch_status();
  }
  const int nb = permute_blocks(S);
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nb), dim3(kPermuteThreads), 0, stream, ids, S, (int)E, block_hist);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  if (nb <= kScanInScatter) {
    hipLaunchKernelGGL(permute_scan_scatter_kernel, dim3(nb), dim3(kPermuteThreads), 0, stream, ids, S, (int)E, nb,
                       block_hist, counts, offsets, sorted_slot, slot_to_row);
    return launch_status();
  }
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, stream, block_hist, nb, (int)E, counts, offsets);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(kPermuteThreads), 0, stream, ids, S, (int)E,
                     block_hist, sorted_slot, slot_to_row);
  return launch_status();
}

moe_status_t launch_topk_permute_small(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, float* w,
                                       int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                                       int32_t* slot_to_row, hipStream_t stream) {
  hipLaunchKernelGGL(topk_permute_small_kernel, dim3(1), dim3(kPermuteThreads), 0, stream, logits, (int)T, (int)E,
                     (int)k, ids, w, counts, offsets, sorted_slot, slot_to_row);
  return launch_status();
}

}  // namespace moe
