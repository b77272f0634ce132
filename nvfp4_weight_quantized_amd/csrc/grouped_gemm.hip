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
//    the token matrix -- no permuted copy -- and staged in LDS per 128-wide K chunk.
//  * B (weights) never goes through LDS: each lane loads 16 bytes of packed nibbles of one weight
//    row per chunk (32 consecutive K) plus their two E4M3 scale bytes and dequantizes them in
//    registers into the bf16 MFMA operand: v_cvt_scalef32_pk_f32_fp4 (scale 1) gives the E2M1
//    values, one fp32 multiply applies the block scale and v_cvt_pk_bf16_f32 packs the result.
//    element * block scale has at most 6 significant bits, so the bf16 operand is exact.
//  * The MFMA reduction order over K is permuted consistently for A and B (lane group q of a
//    16x16x32 fragment owns K range [32q, 32q+32) of the chunk), which makes every lane's weight
//    bytes contiguous; the sum is over the same products.
//  * fp32 accumulation; the per-tensor global scales multiply the accumulators in the epilogue;
//    gate/up workgroups hold matching gate and up columns so h = silu(g)*u is formed in registers.
//  * Groups (experts) are found on the device from the offsets array: no host synchronisation.
//    Workgroups beyond the real tile count exit at once; empty experts cost nothing.
#include "common.h"

namespace moe {
namespace {

constexpr int kBK = 128;        // K chunk
constexpr int kAPad = 8;        // bf16 of padding per LDS row (16 bytes) against bank conflicts
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
// GATE_UP: fragments [0, NB/2) are gate columns, [NB/2, NB) the matching up columns.
template <int MI, int NB, bool GATE_UP>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmProblem p) {
  constexpr int BM = 16 * MI;
  constexpr int COLS_PER_WAVE = GATE_UP ? 16 * (NB / 2) : 16 * NB;   // output columns per wave
  constexpr int BN = 4 * COLS_PER_WAVE;                               // output columns per workgroup
  constexpr int A_ITERS = BM / 16;                                    // 16 rows x 16 x 16B per pass
  __shared__ __attribute__((aligned(16))) uint16_t As[BM][kBK + kAPad];
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
  const int nK = K / kBK;

  // A rows this thread copies: r = tid/16 + 16*it, 16 bytes at column (tid%16)*8 of the chunk
  const uint16_t* arow[A_ITERS];
#pragma unroll
  for (int it = 0; it < A_ITERS; ++it) {
    const int r = (tid >> 4) + 16 * it;
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
  const int acol = (tid & 15) * 8;

  // B rows this lane reads: weight row n for fragment f; lane group q owns K [32q, 32q+32)
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
      n = ntile * (BN) + wave * COLS_PER_WAVE + 16 * fg + nl;
      if (f >= NB / 2) n += p.N;  // up rows follow the gate rows
    } else {
      n = ntile * BN + wave * COLS_PER_WAVE + 16 * f + nl;
    }
    wptr[f] = wbase + (size_t)n * wrow_bytes + 16 * q;
    sptr[f] = sbase + (size_t)n * srow_bytes + 2 * q;
  }

  f32x4 acc[MI][NB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int f = 0; f < NB; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 a_next[A_ITERS];
  uint4 b_next[NB];
  uint16_t s_next[NB];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it)
      a_next[it] = arow[it] ? *reinterpret_cast<const uint4*>(arow[it] + c * kBK + acol) : uint4{0, 0, 0, 0};
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      b_next[f] = *reinterpret_cast<const uint4*>(wptr[f] + (size_t)c * (kBK / 2));
      s_next[f] = *reinterpret_cast<const uint16_t*>(sptr[f] + (size_t)c * (kBK / 16));
    }
  };
  load_chunk(0);

  for (int c = 0; c < nK; ++c) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it)
      *reinterpret_cast<uint4*>(&As[(tid >> 4) + 16 * it][acol]) = a_next[it];
    uint4 bq[NB];
    uint32_t sc[NB];
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      bq[f] = b_next[f];
      sc[f] = s_next[f];
    }
    __syncthreads();
    if (c + 1 < nK) load_chunk(c + 1);

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 bfrag[NB];
#pragma unroll
      for (int f = 0; f < NB; ++f) {
        const uint32_t words[4] = {bq[f].x, bq[f].y, bq[f].z, bq[f].w};
        const float s = (j < 2) ? __builtin_amdgcn_cvt_f32_fp8((int)sc[f], 0)
                                : __builtin_amdgcn_cvt_f32_fp8((int)sc[f], 1);
        bfrag[f] = dequant8(words[j], s);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const bf16x8 afrag = *reinterpret_cast<const bf16x8*>(&As[16 * i + nl][32 * q + 8 * j]);
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

template <int MI, int NB, bool GATE_UP>
moe_status_t launch_cfg(const GemmProblem& p, hipStream_t stream) {
  constexpr int BM = 16 * MI;
  constexpr int BN = GATE_UP ? 4 * 16 * (NB / 2) : 4 * 16 * NB;
  const int NT = p.N / BN;
  // upper bound on m-tiles: every non-empty group adds at most one partial tile
  const long long mt = (p.G > 0 ? (long long)std::min(p.G, p.M) + p.M / BM : 0LL) +
                       (p.has_extra ? (p.M_extra + BM - 1) / BM : 0);
  const long long grid = mt * NT;
  if (grid == 0) return MOE_OK;
  if (grid > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL((grouped_gemm_kernel<MI, NB, GATE_UP>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return launch_status();
}

}  // namespace

moe_status_t launch_grouped_gemm(const GemmProblem& p, hipStream_t stream) {
  const bool gate_up = p.stage == MOE_GEMM_GATE_UP;
  // rows per group on average decides the tile height
  const long long rows = (long long)p.M + (p.has_extra ? p.M_extra : 0);
  const long long groups = (long long)p.G + (p.has_extra ? 1 : 0);
  const long long avg = groups ? rows / groups : 0;
  if (gate_up) {
    if (avg <= 16) return launch_cfg<1, 2, true>(p, stream);
    if (avg <= 64) return launch_cfg<4, 4, true>(p, stream);
    return launch_cfg<8, 4, true>(p, stream);
  }
  const bool wide = (p.N % 256) == 0;
  if (avg <= 16) return launch_cfg<1, 2, false>(p, stream);
  if (avg <= 64) return wide ? launch_cfg<4, 4, false>(p, stream) : launch_cfg<4, 2, false>(p, stream);
  return wide ? launch_cfg<8, 4, false>(p, stream) : launch_cfg<8, 2, false>(p, stream);
}

}  // namespace moe
