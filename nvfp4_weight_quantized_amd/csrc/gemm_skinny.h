// The skinny (few rows per expert: decode-shaped) grouped NVFP4 GEMM tile, shared by the stand-alone
// grouped GEMM kernel and the fused decode kernel, plus the weight-stream helpers the grouped GEMM
// kernels use.  Method: weight-only W4A16, 16-bit activations times 4-bit weights ("vLLM on the
// NVIDIA DGX Spark: A Complete Technical Guide", section 5, Marlin), NVFP4 format of section 6.1.
#pragma once

#include "common.h"
#include "gemm_tiles.h"

namespace moe {
namespace {

constexpr int kAPad = 8;              // bf16 of padding per LDS row (16 bytes) against bank conflicts
constexpr int kSkinnyThreads = 256;   // 4 waves

// The 8 E2M1 codes of one dword as bf16, unscaled (exact: every E2M1 value is a bf16).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t q) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// E4M3 block scale held in byte j (0..3) of a scale dword (the byte select must fold to a constant).
__device__ __forceinline__ float e4m3_byte(uint32_t sc, int j) {
  switch (j) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)sc, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)sc, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)sc, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)sc, 3);
  }
}

// Byte offsets, within an expert's tiles, of the 16 nibble bytes and the scale dword of this lane.
__device__ __forceinline__ int w_lane_offset(int lane) { return 16 * lane; }
__device__ __forceinline__ int s_lane_offset(int lane) { return 8 * (lane & 15) + 4 * ((lane >> 4) >> 1); }

// Streaming (non-temporal) loads for weight bytes that are read once per pass.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ uint32_t load_stream4(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// ------------------------------------------------------------------------------------------
// Skinny tiles (a few rows per group, the decode shape): weight-bandwidth bound, so the work per
// weight byte is what counts.  Up to 8 rows per tile.
//  * The activations are the MFMA's first operand and the weights its second, unscaled (one
//    conversion per two codes); the E4M3 block scale is applied to the fp32 MFMA result instead,
//    one FMA per useful accumulator register, not one multiply per weight element.
//  * For that, each MFMA must sum over a single 16-element scale group.  A 16x16x32 step covers
//    two groups (K [0,16) in lanes q = 0, 1 and K [16,32) in lanes q = 2, 3 of the weight tile), so
//    every token appears twice in the 16-row activation fragment: at row 4(t%2) + t/2 with the
//    second group's columns zeroed and at that row + 8 with the first group's columns zeroed.
//    Accumulator register r of lane (q, n) then holds token 2r + q%2, weight row n, scale group
//    2j + q/2 -- one scale per lane per step, the dword the weight tile layout already gives the
//    lane -- and the two groups' sums are added across lanes 32 apart at the end.
//  * Tokens 0-1 need one accumulator register per weight fragment, 2-3 two, 4-7 four: the main
//    loop is instantiated for 1, 2 and 4 and the tile's row count picks one.
//  * The zeroed halves of the LDS fragment are cleared once; each K chunk overwrites only the
//    token columns.
constexpr int kSkinnyRows = 8;

template <int N>
struct RegsC {
  static constexpr int value = N;
};

// LDS of one skinny tile: the 16-row activation fragment of a K chunk and the tile lookup.
template <int BK>
struct SkinnyLds {
  __attribute__((aligned(16))) uint16_t As[16 * (BK + kAPad)];
  TileInfo tile;
  int tile_ok;
};

// Output columns of one skinny workgroup tile.
template <int NB, bool GATE_UP>
constexpr int skinny_bn() {
  return 4 * (GATE_UP ? 16 * (NB / 2) : 16 * NB);
}

// Output store of the skinny epilogue.  DEVICE_COHERENT: written through to device-coherent memory
// (agent-scope store), so that a workgroup on another XCD can read it once the tile's completion is
// signalled, without a write-back of this XCD's L2.
template <bool DEVICE_COHERENT>
__device__ __forceinline__ void store_out(uint16_t* dst, uint16_t v) {
  if constexpr (DEVICE_COHERENT) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *dst = v;
}

// One skinny tile: m-tile `mtile` (8-row tiles over the groups, the extra group's first) times
// output-column tile `ntile`, by the whole 256-thread workgroup.  Returns false (having written
// nothing) when the m-tile does not exist.  Every thread of the workgroup must call it.
template <int NB, int BK, bool GATE_UP, bool DEVICE_COHERENT = false>
__device__ __forceinline__ bool skinny_tile(const GemmProblem& p, int mtile, int ntile, SkinnyLds<BK>& L) {
  constexpr int BM = kSkinnyRows;
  constexpr int NS = BK / 128;                                       // weight tiles per fragment per chunk
  constexpr int COLS_PER_WAVE = GATE_UP ? 16 * (NB / 2) : 16 * NB;
  constexpr int BN = 4 * COLS_PER_WAVE;
  constexpr int LDS_ROW = BK + kAPad;
  constexpr int A_TPR = BK / 8;                                      // threads per token row (16 bytes each)
  constexpr int A_RPP = kSkinnyThreads / A_TPR;                      // token rows per pass
  constexpr int A_ITERS = (BM + A_RPP - 1) / A_RPP;
  static_assert(BK % 128 == 0 && BK <= 512 && A_RPP * A_ITERS >= BM, "chunk layout");
  uint16_t* As = L.As;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  if (wave == 0) {
    const bool ok = find_tile<BM>(p, mtile, &L.tile);
    if (lane == 0) L.tile_ok = ok ? 1 : 0;
  }
  for (int i = tid; i < 16 * LDS_ROW / 8; i += kSkinnyThreads) reinterpret_cast<uint4*>(As)[i] = uint4{0, 0, 0, 0};
  __syncthreads();
  if (!L.tile_ok) return false;
  const TileInfo ti = L.tile;
  const GemmBank& bank = ti.extra ? p.extra : p.bank;
  const int K = p.K;
  const int nK = K / BK;
  const int ktiles = K / 128;

  // token rows this thread copies: t = tid/A_TPR + A_RPP*it, 16 bytes at column acol, into
  // fragment row 4(t%2) + t/2 (+8 when the column lies in the second group of its 32-wide step)
  const int acol = (tid % A_TPR) * 8;
  const uint16_t* arow[A_ITERS];
  int alds[A_ITERS];
#pragma unroll
  for (int it = 0; it < A_ITERS; ++it) {
    const int t = tid / A_TPR + A_RPP * it;
    arow[it] = nullptr;
    alds[it] = 0;
    if (t < ti.rows) {
      const int R = ti.a_row0 + t;
      if (ti.extra) {
        arow[it] = p.a_extra + (size_t)R * K;
      } else {
        const int src = p.row_index ? p.row_index[R] / p.row_divisor : R;
        arow[it] = p.a + (size_t)src * K;
      }
      alds[it] = (4 * (t & 1) + (t >> 1) + ((acol & 16) ? 8 : 0)) * LDS_ROW + acol;
    }
  }

  const int q = lane >> 4;
  const int nl = lane & 15;
  const size_t rows_per_expert = GATE_UP ? 2 * (size_t)p.N : (size_t)p.N;
  const uint8_t* wexp = bank.w + (size_t)ti.group * rows_per_expert * (size_t)(K / 2) + w_lane_offset(lane);
  const uint8_t* sexp = bank.ws + (size_t)ti.group * rows_per_expert * (size_t)(K / 16) + s_lane_offset(lane);
  const uint8_t* wptr[NB];
  const uint8_t* sptr[NB];
#pragma unroll
  for (int f = 0; f < NB; ++f) {
    const size_t t0 = (size_t)frag_row_block<NB, GATE_UP, BN, COLS_PER_WAVE>(f, ntile, wave, p.N) * ktiles;
    wptr[f] = wexp + t0 * 1024;
    sptr[f] = sexp + t0 * 128;
  }

  float acc[NB][4];
#pragma unroll
  for (int f = 0; f < NB; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[f][r] = 0.f;

  auto run = [&](auto regs_const) {
    constexpr int RG = decltype(regs_const)::value;   // accumulator registers holding tokens
    uint4 a_next[A_ITERS];
    uint4 b_next[NB][NS];
    uint32_t s_next[NB][NS];
    auto load_chunk = [&](int c) {
#pragma unroll
      for (int it = 0; it < A_ITERS; ++it)
        if (arow[it]) a_next[it] = *reinterpret_cast<const uint4*>(arow[it] + (size_t)c * BK + acol);
#pragma unroll
      for (int f = 0; f < NB; ++f)
#pragma unroll
        for (int v = 0; v < NS; ++v) {
          const size_t t = (size_t)c * NS + v;
          b_next[f][v] = load_stream16(wptr[f] + t * 1024);
          s_next[f][v] = load_stream4(sptr[f] + t * 128);
        }
    };
    load_chunk(0);
    const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nK; ++c) {
      __syncthreads();
#pragma unroll
      for (int it = 0; it < A_ITERS; ++it)
        if (arow[it]) *reinterpret_cast<uint4*>(As + alds[it]) = a_next[it];
      uint4 bq[NB][NS];
      uint32_t sc[NB][NS];
#pragma unroll
      for (int f = 0; f < NB; ++f)
#pragma unroll
        for (int v = 0; v < NS; ++v) {
          bq[f][v] = b_next[f][v];
          sc[f][v] = s_next[f][v];
        }
      __syncthreads();
      if (c + 1 < nK) load_chunk(c + 1);
#pragma unroll
      for (int v = 0; v < NS; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 xfrag = *reinterpret_cast<const bf16x8*>(As + nl * LDS_ROW + 128 * v + 32 * j + 8 * q);
#pragma unroll
          for (int f = 0; f < NB; ++f) {
            const uint32_t words[4] = {bq[f][v].x, bq[f][v].y, bq[f][v].z, bq[f][v].w};
            const f32x4 part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xfrag, fp4x8_to_bf16(words[j]), zero, 0, 0, 0);
            const float s = e4m3_byte(sc[f][v], j);
#pragma unroll
            for (int r = 0; r < RG; ++r) acc[f][r] = fmaf(s, part[r], acc[f][r]);
          }
          // one step's MFMA results at a time (bounds the live registers)
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  };
  if (ti.rows <= 2) run(RegsC<1>{});
  else if (ti.rows <= 4) run(RegsC<2>{});
  else run(RegsC<4>{});

  // first scale group's sums (lanes q < 2) plus the second's (32 lanes above)
#pragma unroll
  for (int f = 0; f < NB; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[f][r] += __shfl_xor(acc[f][r], 32);
  if (q >= 2) return true;
  const float* gs = bank.gs + (size_t)ti.group * bank.gs_per_expert;
  const int col = ntile * BN + wave * COLS_PER_WAVE + nl;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 2 * r + q;
    if (t >= ti.rows) continue;
    uint16_t* orow = p.out + (size_t)(ti.row0 + t) * p.N + col;
    if (GATE_UP) {
      const float dg = gs[0] * act_gscale(p), du = gs[1] * act_gscale(p);
#pragma unroll
      for (int f = 0; f < NB / 2; ++f)
        store_out<DEVICE_COHERENT>(orow + 16 * f, f32_to_bf16(silu(acc[f][r] * dg) * (acc[f + NB / 2][r] * du)));
    } else {
      const float dd = gs[0] * act_gscale(p);
#pragma unroll
      for (int f = 0; f < NB; ++f) store_out<DEVICE_COHERENT>(orow + 16 * f, f32_to_bf16(acc[f][r] * dd));
    }
  }
  return true;
}

}  // namespace
}  // namespace moe
