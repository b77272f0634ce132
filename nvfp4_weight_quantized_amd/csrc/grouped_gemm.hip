// Grouped NVFP4 x bf16 GEMMs of the MoE layer (S4 gate/up with SiLU(gate)*up, S5 down), gfx950.
//
// Method: weight-only W4A16 -- 16-bit activations times 4-bit weights that are dequantized to
// 16-bit inside the GEMM ("vLLM on the NVIDIA DGX Spark: A Complete Technical Guide", section 5,
// Marlin), on the NVFP4 format of section 6.1 (E2M1 pairs per byte, one E4M3 scale per 16
// elements along K, one fp32 global scale per tensor).  SiLU(gate)*up between the GEMMs as in the
// fused MoE of section 4.
//
// CDNA4 design:
//  * A (activation rows, bf16) is gathered row by row through the sorted slot list straight from
//    the token matrix -- no permuted copy -- and staged in LDS per K chunk (BK = 128 for tall
//    tiles, up to 512 for the 16-row tiles of decode-sized groups).
//  * B (weights) never goes through LDS: each lane loads BK/8 contiguous bytes of packed nibbles
//    of one weight row per chunk plus their BK/64 E4M3 scale bytes and dequantizes them in
//    registers into the bf16 MFMA operand: v_cvt_scalef32_pk_f32_fp4 (scale 1) gives the E2M1
//    values, one fp32 multiply applies the block scale and v_cvt_pk_bf16_f32 packs the result.
//    element * block scale has at most 6 significant bits, so the bf16 operand is exact.
//  * The MFMA reduction order over K is permuted consistently for A and B (lane group q of a
//    16x16x32 fragment owns K range [q*BK/4, (q+1)*BK/4) of the chunk), which makes every lane's
//    weight bytes contiguous; the sum is over the same products.
//  * fp32 accumulation; the per-tensor global scales multiply the accumulators in the epilogue;
//    gate/up workgroups hold matching gate and up columns so h = silu(g)*u is formed in registers.
//  * Groups (experts) are found on the device from the offsets array: no host synchronisation.
//    Workgroups beyond the real tile count exit at once; empty experts cost nothing.
#include "common.h"

namespace moe {
namespace {

constexpr int kAPad = 8;       // bf16 of padding per LDS row (16 bytes) against bank conflicts
constexpr int kThreads = 256;   // 4 waves

struct TileInfo {
  int group;     // expert index in its bank
  int row0;      // first output row of the tile (global row index in the output)
  int rows;      // valid rows (<= BM)
  int a_row0;    // first A row (for extra / identity rows) or first sorted row
  int extra;     // 1: shared-expert group
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// Dequantize 8 packed E2M1 codes (one dword, element order = nibble order) times scale s.
__device__ __forceinline__ bf16x8 dequant8(uint32_t q, float s) {
  const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
  const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
  const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
  const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
  bf16x8 r;
  r[0] = (__bf16)(p0[0] * s);
  r[1] = (__bf16)(p0[1] * s);
  r[2] = (__bf16)(p1[0] * s);
  r[3] = (__bf16)(p1[1] * s);
  r[4] = (__bf16)(p2[0] * s);
  r[5] = (__bf16)(p2[1] * s);
  r[6] = (__bf16)(p3[0] * s);
  r[7] = (__bf16)(p3[1] * s);
  return r;
}

// Find the tile `mtile` (numbered over the groups in order, then the extra group).  Wave 0 only.
template <int BM>
__device__ bool find_tile(const GemmProblem& p, int mtile, TileInfo* out) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  // counts of up to 1024 groups, loaded together
  int cnt[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int g = 64 * i + lane;
    cnt[i] = (g < p.G) ? (p.offsets[g + 1] - p.offsets[g]) : 0;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (64 * i >= p.G) break;
    const int g = 64 * i + lane;
    const int t = (cnt[i] + BM - 1) / BM;
    int incl = t;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const int excl = incl - t;
    const bool hit = (g < p.G) && (t > 0) && (carry + excl <= mtile) && (mtile < carry + incl);
    const uint64_t m = __ballot(hit);
    if (m) {
      const int h = __ffsll((unsigned long long)m) - 1;
      const int within = mtile - carry - __shfl(excl, h);
      const int gcount = __shfl(cnt[i], h);
      if (lane == 0) {
        const int gstart = p.offsets[64 * i + h];
        out->group = 64 * i + h;
        out->row0 = gstart + within * BM;
        out->a_row0 = gstart + within * BM;
        out->rows = min(BM, gcount - within * BM);
        out->extra = 0;
      }
      return true;
    }
    carry += __shfl(incl, 63);
  }
  if (p.has_extra) {
    const int xt = (p.M_extra + BM - 1) / BM;
    const int within = mtile - carry;
    if (within < xt) {
      if (lane == 0) {
        out->group = 0;
        out->row0 = p.M + within * BM;
        out->a_row0 = within * BM;
        out->rows = min(BM, p.M_extra - within * BM);
        out->extra = 1;
      }
      return true;
    }
  }
  return false;
}

// MI: 16-row A fragments per wave (BM = 16*MI).  NB: 16-column B fragments per wave.
// BK: K chunk (128, 256 or 512); lane group q of a fragment owns K range [q*BK/4, (q+1)*BK/4) of
// the chunk, i.e. BK/8 contiguous weight bytes and BK/64 contiguous scale bytes of its row.
// GATE_UP: fragments [0, NB/2) are gate columns, [NB/2, NB) the matching up columns.
template <int MI, int NB, int BK, bool GATE_UP>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmProblem p) {
  constexpr int BM = 16 * MI;
  constexpr int COLS_PER_WAVE = GATE_UP ? 16 * (NB / 2) : 16 * NB;   // output columns per wave
  constexpr int BN = 4 * COLS_PER_WAVE;                               // output columns per workgroup
  constexpr int LANE_K = BK / 4;        // K values per lane per chunk
  constexpr int NV = LANE_K / 32;       // 16-byte nibble loads per lane per fragment per chunk
  constexpr int LANE_S = LANE_K / 16;   // scale bytes per lane per chunk (2, 4 or 8)
  constexpr int STEPS = BK / 32;        // MFMA k-steps per chunk
  constexpr int A_TPR = BK / 8;         // threads per A row (16 bytes each)
  constexpr int A_RPP = kThreads / A_TPR;   // A rows per pass
  constexpr int A_ITERS = BM / A_RPP;       // passes
  static_assert(BM % A_RPP == 0, "A tile must be a whole number of passes");
  static_assert(LANE_S == 2 || LANE_S == 4 || LANE_S == 8, "BK must be 128, 256 or 512");
  __shared__ __attribute__((aligned(16))) uint16_t As[BM][BK + kAPad];
  __shared__ TileInfo tile;
  __shared__ int tile_ok;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int NT = p.N / BN;
  const int mtile = blockIdx.x / NT;
  const int ntile = blockIdx.x - mtile * NT;

  if (wave == 0) {
    const bool ok = find_tile<BM>(p, mtile, &tile);
    if (lane == 0) tile_ok = ok ? 1 : 0;
  }
  __syncthreads();
  if (!tile_ok) return;
  const TileInfo ti = tile;
  const GemmBank& bank = ti.extra ? p.extra : p.bank;
  const int K = p.K;
  const int nK = K / BK;

  // A rows this thread copies: r = tid/A_TPR + A_RPP*it, 16 bytes at column (tid%A_TPR)*8
  const uint16_t* arow[A_ITERS];
#pragma unroll
  for (int it = 0; it < A_ITERS; ++it) {
    const int r = tid / A_TPR + A_RPP * it;
    arow[it] = nullptr;
    if (r < ti.rows) {
      const int R = ti.a_row0 + r;
      if (ti.extra) {
        arow[it] = p.a_extra + (size_t)R * K;
      } else {
        const int src = p.row_index ? p.row_index[R] / p.row_divisor : R;
        arow[it] = p.a + (size_t)src * K;
      }
    }
  }
  const int acol = (tid % A_TPR) * 8;

  // B rows this lane reads: weight row n for fragment f
  const int q = lane >> 4;
  const int nl = lane & 15;
  const size_t wrow_bytes = (size_t)K / 2;
  const size_t srow_bytes = (size_t)K / 16;
  const size_t rows_per_expert = GATE_UP ? 2 * (size_t)p.N : (size_t)p.N;
  const uint8_t* wbase = bank.w + (size_t)ti.group * rows_per_expert * wrow_bytes;
  const uint8_t* sbase = bank.ws + (size_t)ti.group * rows_per_expert * srow_bytes;
  const uint8_t* wptr[NB];
  const uint8_t* sptr[NB];
#pragma unroll
  for (int f = 0; f < NB; ++f) {
    int n;
    if (GATE_UP) {
      const int fg = (f < NB / 2) ? f : f - NB / 2;
      n = ntile * BN + wave * COLS_PER_WAVE + 16 * fg + nl;
      if (f >= NB / 2) n += p.N;  // up rows follow the gate rows
    } else {
      n = ntile * BN + wave * COLS_PER_WAVE + 16 * f + nl;
    }
    wptr[f] = wbase + (size_t)n * wrow_bytes + (LANE_K / 2) * q;
    sptr[f] = sbase + (size_t)n * srow_bytes + LANE_S * q;
  }

  f32x4 acc[MI][NB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int f = 0; f < NB; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 a_next[A_ITERS];
  uint4 b_next[NB][NV];
  uint32_t s_next[NB][2];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it)
      a_next[it] = arow[it] ? *reinterpret_cast<const uint4*>(arow[it] + (size_t)c * BK + acol) : uint4{0, 0, 0, 0};
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      const uint8_t* wp = wptr[f] + (size_t)c * (BK / 2);
#pragma unroll
      for (int v = 0; v < NV; ++v) b_next[f][v] = *reinterpret_cast<const uint4*>(wp + 16 * v);
      const uint8_t* sp = sptr[f] + (size_t)c * (BK / 16);
      if constexpr (LANE_S == 2) {
        s_next[f][0] = *reinterpret_cast<const uint16_t*>(sp);
        s_next[f][1] = 0;
      } else if constexpr (LANE_S == 4) {
        s_next[f][0] = *reinterpret_cast<const uint32_t*>(sp);
        s_next[f][1] = 0;
      } else {
        const uint2 sv = *reinterpret_cast<const uint2*>(sp);
        s_next[f][0] = sv.x;
        s_next[f][1] = sv.y;
      }
    }
  };
  load_chunk(0);

  for (int c = 0; c < nK; ++c) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it)
      *reinterpret_cast<uint4*>(&As[tid / A_TPR + A_RPP * it][acol]) = a_next[it];
    uint4 bq[NB][NV];
    uint32_t sc[NB][2];
#pragma unroll
    for (int f = 0; f < NB; ++f) {
#pragma unroll
      for (int v = 0; v < NV; ++v) bq[f][v] = b_next[f][v];
      sc[f][0] = s_next[f][0];
      sc[f][1] = s_next[f][1];
    }
    __syncthreads();
    if (c + 1 < nK) load_chunk(c + 1);

#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
      bf16x8 bfrag[NB];
#pragma unroll
      for (int f = 0; f < NB; ++f) {
        const uint4 bv = bq[f][j / 4];
        const uint32_t words[4] = {bv.x, bv.y, bv.z, bv.w};
        const int sb = j / 2;   // scale byte of this k-step within the lane's scale bytes
        const uint32_t sw = sc[f][sb / 4];
        float s;
        switch (sb % 4) {
          case 0: s = __builtin_amdgcn_cvt_f32_fp8((int)sw, 0); break;
          case 1: s = __builtin_amdgcn_cvt_f32_fp8((int)sw, 1); break;
          case 2: s = __builtin_amdgcn_cvt_f32_fp8((int)sw, 2); break;
          default: s = __builtin_amdgcn_cvt_f32_fp8((int)sw, 3); break;
        }
        bfrag[f] = dequant8(words[j % 4], s);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const bf16x8 afrag = *reinterpret_cast<const bf16x8*>(&As[16 * i + nl][LANE_K * q + 8 * j]);
#pragma unroll
        for (int f = 0; f < NB; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag[f], acc[i][f], 0, 0, 0);
      }
    }
  }

  // epilogue
  const float* gs = bank.gs + (size_t)ti.group * bank.gs_per_expert;
  if (GATE_UP) {
    const float dg = gs[0], du = gs[1];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int f = 0; f < NB / 2; ++f) {
        const int col = ntile * BN + wave * COLS_PER_WAVE + 16 * f + nl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * i + 4 * q + r;
          if (row < ti.rows) {
            const float g = acc[i][f][r] * dg;
            const float u = acc[i][f + NB / 2][r] * du;
            p.out[(size_t)(ti.row0 + row) * p.N + col] = f32_to_bf16(silu(g) * u);
          }
        }
      }
  } else {
    const float dd = gs[0];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int f = 0; f < NB; ++f) {
        const int col = ntile * BN + wave * COLS_PER_WAVE + 16 * f + nl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * i + 4 * q + r;
          if (row < ti.rows) p.out[(size_t)(ti.row0 + row) * p.N + col] = f32_to_bf16(acc[i][f][r] * dd);
        }
      }
  }
}

template <int MI, int NB, int BK, bool GATE_UP>
moe_status_t launch_cfg(const GemmProblem& p, hipStream_t stream) {
  constexpr int BM = 16 * MI;
  constexpr int BN = GATE_UP ? 4 * 16 * (NB / 2) : 4 * 16 * NB;
  if (p.N % BN != 0 || p.K % BK != 0) return MOE_ERR_INVALID_ARGUMENT;
  const int NT = p.N / BN;
  // upper bound on m-tiles: every non-empty group adds at most one partial tile
  const long long mt = (p.G > 0 ? (long long)std::min(p.G, p.M) + p.M / BM : 0LL) +
                       (p.has_extra ? (p.M_extra + BM - 1) / BM : 0);
  const long long grid = mt * NT;
  if (grid == 0) return MOE_OK;
  if (grid > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL((grouped_gemm_kernel<MI, NB, BK, GATE_UP>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return launch_status();
}

// Few rows per expert: 16-row tiles and the widest K chunk the reduction length allows, so that
// each lane streams 64 contiguous weight bytes per fragment per chunk.
template <bool GATE_UP>
moe_status_t launch_small(const GemmProblem& p, hipStream_t stream) {
  if (p.K % 512 == 0) return launch_cfg<1, 2, 512, GATE_UP>(p, stream);
  if (p.K % 256 == 0) return launch_cfg<1, 2, 256, GATE_UP>(p, stream);
  return launch_cfg<1, 2, 128, GATE_UP>(p, stream);
}

}  // namespace

moe_status_t launch_grouped_gemm(const GemmProblem& p, hipStream_t stream) {
  const bool gate_up = p.stage == MOE_GEMM_GATE_UP;
  // rows per group on average decides the tile height
  const long long rows = (long long)p.M + (p.has_extra ? p.M_extra : 0);
  const long long groups = (long long)p.G + (p.has_extra ? 1 : 0);
  const long long avg = groups ? rows / groups : 0;
  if (gate_up) {
    if (avg <= 16) return launch_small<true>(p, stream);
    if (avg <= 64) return launch_cfg<4, 4, 128, true>(p, stream);
    return launch_cfg<8, 4, 128, true>(p, stream);
  }
  const bool wide = (p.N % 256) == 0;
  if (avg <= 16) return launch_small<false>(p, stream);
  if (avg <= 64) return wide ? launch_cfg<4, 4, 128, false>(p, stream) : launch_cfg<4, 2, 128, false>(p, stream);
  return wide ? launch_cfg<8, 4, 128, false>(p, stream) : launch_cfg<8, 2, 128, false>(p, stream);
}

}  // namespace moe
