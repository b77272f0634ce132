// Tile bookkeeping shared by the grouped GEMM kernels (W4A16 and W4A4): the tile list over the
// expert groups, the weight fragments of a wave, and the bf16 epilogue with SiLU(gate)*up.
#pragma once

#include <cstddef>
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

struct TileInfo {
  int group;     // expert index in its bank
  int row0;      // first output row of the tile (global row index in the output)
  int rows;      // valid rows (<= BM)
  int a_row0;    // first A row (for extra / identity rows) or first sorted row
  int extra;     // 1: shared-expert group
};

// SiLU(g) = g / (1 + e^-g) with the hardware base-2 exponential and reciprocal (v_exp_f32, v_rcp_f32,
// about 1 ulp each): a handful of instructions instead of the library exponential and an IEEE
// division (about 25 VALU instructions per output, 10% of the prefill gate/up GEMM as its
// epilogue).  The result is rounded to bf16 (8 significant bits) right after.  Limits: e^-g
// overflows to +inf for g < -88.7 and the reciprocal gives 0, so SiLU -> -0; g = +inf gives +inf,
// and g = -inf or NaN give NaN, as the exact formula does.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
}

constexpr int kXcds = 8;

// This lane's index in its wave, computed where it is used (the mask count is opaque to the
// optimizer, so no register holds it, or values derived from it, across the code in between).
__device__ __forceinline__ int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

// Tile `mtile`: the extra group's tiles come first (the shared expert, every token: the longest
// group, started early), then each group's in order.  Wave 0 only.  Lane i owns the contiguous
// groups [i*gpl, (i+1)*gpl) (gpl = ceil(G/64) <= 16): one scan of the lanes' tile counts finds the
// owning lane, which walks its groups.  `span` (optional) receives the tile's index within its
// group and the group's row count.
template <int BM, class P>
__device__ bool find_tile(const P& p, int mtile, TileInfo* out, int2* span = nullptr) {
  const int lane = threadIdx.x & 63;
  if (p.has_extra) {
    const int xt = (p.M_extra + BM - 1) / BM;
    if (mtile < xt) {
      if (lane == 0) {
        out->group = 0;
        out->row0 = p.M + mtile * BM;
        out->a_row0 = mtile * BM;
        out->rows = min(BM, p.M_extra - mtile * BM);
        out->extra = 1;
        if (span) *span = int2{mtile, p.M_extra};
      }
      return true;
    }
    mtile -= xt;
  }
  const int gpl = (p.G + 63) >> 6;
  const int g0 = lane * gpl;
  int start[17];
#pragma unroll
  for (int i = 0; i <= 16; ++i) start[i] = (i <= gpl && g0 + i <= p.G) ? p.offsets[g0 + i] : 0;
  int t = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (i < gpl && g0 + i < p.G) t += (start[i + 1] - start[i] + BM - 1) / BM;
  int incl = t;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const int excl = incl - t;
  const uint64_t m = __ballot(excl <= mtile && mtile < incl);
  if (!m) return false;
  if (lane == __ffsll((unsigned long long)m) - 1) {
    int first = excl;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i >= gpl || g0 + i >= p.G) break;
      const int cnt = start[i + 1] - start[i];
      const int ti = (cnt + BM - 1) / BM;
      if (mtile < first + ti) {
        const int within = mtile - first;
        out->group = g0 + i;
        out->row0 = start[i] + within * BM;
        out->a_row0 = start[i] + within * BM;
        out->rows = min(BM, cnt - within * BM);
        out->extra = 0;
        if (span) *span = int2{within, cnt};
        break;
      }
      first += ti;
    }
  }
  return true;
}

// Wave 0: number of BM-row tiles over the groups (+ extra group).
template <int BM, class P>
__device__ int count_tiles(const P& p) {
  const int lane = threadIdx.x & 63;
  int t = 0;
  for (int g = lane; g < p.G; g += 64) t += (p.offsets[g + 1] - p.offsets[g] + BM - 1) / BM;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
  if (p.has_extra) t += (p.M_extra + BM - 1) / BM;
  return t;
}

// Weight-row block (16 rows) of B fragment f of `wave` in output-column tile `ntile`.
template <int NB, bool GATE_UP, int BN, int COLS_PER_WAVE>
__device__ __forceinline__ int frag_row_block(int f, int ntile, int wave, int N) {
  int n;
  if (GATE_UP) {
    const int fg = (f < NB / 2) ? f : f - NB / 2;
    n = ntile * BN + wave * COLS_PER_WAVE + 16 * fg;
    if (f >= NB / 2) n += N;  // up rows follow the gate rows
  } else {
    n = ntile * BN + wave * COLS_PER_WAVE + 16 * f;
  }
  return n >> 4;
}

// Activation global scale of a problem: the W4A16 problems' (act_gscale), 1 for the MX W4A4 one.
__device__ __forceinline__ float epilogue_act_gscale(const GemmProblem& p) { return act_gscale(p); }
template <class P>
__device__ __forceinline__ float epilogue_act_gscale(const P&) { return 1.f; }
// The fp16 h path of a problem (GemmProblem::h16; never for the MX W4A4 one).
__device__ __forceinline__ bool epilogue_h16(const GemmProblem& p) { return p.h16 != 0; }
template <class P>
__device__ __forceinline__ bool epilogue_h16(const P&) { return false; }
__device__ __forceinline__ int32_t* epilogue_hshift_out(const GemmProblem& p) { return p.hshift_out; }
template <class P>
__device__ __forceinline__ int32_t* epilogue_hshift_out(const P&) { return nullptr; }

// Epilogue: scale the accumulators by the global scale(s), SiLU(gate)*up for gate/up, store bf16.
// acc[i][f] holds, in lane l = 16q + n, output row 16i + n and the four columns 4q..4q+3 of
// fragment f's 16 columns (gate/up: fragments NB/2.. hold the up columns of fragments 0..).
// GSCALE: the bank carries fp32 global scales (NVFP4); otherwise the scale is 1.
// rshift (optional): per tile row, the powers of two of the fp16 operand rows.  Gate/up: the
// token row was scaled by 2^xs, xs = (int16_t)rshift[row], and the sums are scaled back by 2^-xs
// (exact) before SiLU; with the fp16 h path (p.h16), h = bf16(silu(g) u) is stored as fp16 after
// scaling by 2^hs, hs = rshift[row] >> 16 (folded into u's scale: power-of-two scaling commutes with
// the bf16 rounding), and the column-tile-0 workgroup records hs in p.hshift_out[row of h].  Down
// (fp16 h): h row `row` was scaled by 2^rshift[row]; the sums are scaled back by 2^-rshift[row].
// These powers of two enter the global scales (one multiply per value) wherever the scaled global
// scale stays a normal number; otherwise the row block applies them after the product.
// RBE (default MI): the 16-row blocks that can hold rows of the tile; blocks past it are not read,
// so a caller that never touched their accumulators need not keep them.
// epilogue_at takes the weight global scales of the tile's expert (g0: gate or down, g1: up; 1
// without) and the lane and wave indices from the caller.
template <int MI, int NB, bool GATE_UP, int BN, int COLS_PER_WAVE, class P, int RBE = MI, class RS = std::nullptr_t>
__device__ __forceinline__ void epilogue_at(const P& p, float g0, float g1, const TileInfo& ti, int ntile,
                                            const f32x4 (&acc)[MI][NB], int mtile, RS rshift, IntC<RBE>,
                                            int lane, int wave) {
  // the row powers of two are there exactly when the caller passes a pointer (nullptr: none), so
  // that their use is decided at compile time
  constexpr bool kRS = !std::is_same<RS, std::nullptr_t>::value;
  const int q = lane >> 4, nl = lane & 15;
  const float da = epilogue_act_gscale(p);
  // output fragments per wave (16 columns each) and their first column
  constexpr int NF = GATE_UP ? NB / 2 : NB;
  const int colw = ntile * BN + wave * COLS_PER_WAVE;
  // Fragments are stored in pairs (f, f + 1), 16 bytes per lane: v_permlane16_swap exchanges the
  // pair's packed values between the quarters q and q ^ 1 of the wave (lanes 16 apart), after which
  // lane (q, n) holds the eight consecutive columns of row n starting pc columns after the pair's
  // first: quarter 0 the first fragment's columns 0..7, quarter 2 its 8..15, quarters 1 and 3 the
  // second fragment's 0..7 and 8..15.  The four lanes of a row then write its 64 bytes with one
  // store instruction (the tiled layout's 16-byte lane slots, whole), instead of two with 8 bytes
  // per lane and 32 per row; fewer, wider stores retire sooner, and the direct loads of the next
  // chunks wait behind them (the memory counter counts stores).  An odd last fragment is stored
  // 8 bytes per lane as before.  The swap runs in every lane, rows past the tile's included.
  const int pc = 16 * (q & 1) + 8 * (q >> 1);
  auto pack4 = [](float a, float b, float c, float d) { return uint2{f32x2_to_bf16x2(a, b), f32x2_to_bf16x2(c, d)}; };
  // the bf16 rounding of each value, as fp16 (exact for every value of at least 2^-17 and below 2^16;
  // smaller ones round to nearest even on the fp16 subnormal grid): per pair one bf16 pair
  // conversion, the two halves back to fp32, one fp16 pair conversion (v_cvt_pk_f16_f32)
  auto pack4h = [](float a, float b, float c, float d) {
    auto pair = [](float x, float y) {
      const uint32_t bb = f32x2_to_bf16x2(x, y);
      typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
      const f32x2 v = {__uint_as_float(bb << 16), __uint_as_float(bb & 0xFFFF0000u)};
      return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
    };
    return uint2{pair(a, b), pair(c, d)};
  };
  // A row's power of two folded into a scale (one multiply per value instead of a multiply and an
  // ldexp) gives the same roundings wherever the folded scale is a normal number (or the scale is 0):
  // a product is then rounded once either way.  A wave takes the folded form for a row block only
  // when that holds in all its lanes.
  auto foldable = [](float folded, float scale) { return __builtin_isnormal(folded) || scale == 0.f; };
  const bool h16 = kRS && epilogue_h16(p);
  // address of column col (of this lane's row) in block i
  auto dst = [&](int i, int row, int col) -> uint16_t* {
    if (GATE_UP && p.out_tiled) {
      // tiled layout: column col -> chunk col/128, step (col%128)/32, lane slot (col%32)/8
      const int kk = col & 127;
      const size_t byte = ((size_t)(mtile * (p.N >> 7) + (col >> 7)) * 32 + 4 * i + (kk >> 5)) * 1024 +
                          (size_t)(16 * (((kk >> 3) & 3) * 16 + nl) + 2 * (kk & 7));
      return p.out_tiled + byte / 2;
    }
    return p.out + (size_t)(ti.row0 + row) * p.N + col;
  };
#pragma unroll
  for (int i = 0; i < RBE; ++i) {
    const int row = 16 * i + nl;
    const bool valid = row < ti.rows;
    uint2 v[NF];
    if (GATE_UP) {
      const float dg = g0 * da, du = g1 * da;
      int rs = 0;
      if constexpr (kRS) rs = rshift[row];
      const int xs = (int)(int16_t)rs;
      const int hs = h16 ? rs >> 16 : 0;
      auto store_h = [&](auto gate, auto up) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = silu(gate(acc[i][f][r])) * up(acc[i][f + NF][r]);
          v[f] = h16 ? pack4h(h[0], h[1], h[2], h[3]) : pack4(h[0], h[1], h[2], h[3]);
        }
      };
      if constexpr (kRS) {
        const float dgr = ldexpf(dg, -xs), dur = ldexpf(du, hs - xs);
        if (__builtin_amdgcn_ballot_w64(!(foldable(dgr, dg) && foldable(dur, du))) == 0)
          store_h([&](float a) { return a * dgr; }, [&](float a) { return a * dur; });
        else
          store_h([&](float a) { return ldexpf(a * dg, -xs); }, [&](float a) { return ldexpf(a * du, hs - xs); });
      } else {
        store_h([&](float a) { return a * dg; }, [&](float a) { return a * du; });
      }
      if (h16 && ntile == 0 && wave == 0 && q == 0 && valid) epilogue_hshift_out(p)[ti.row0 + row] = hs;
    } else {
      const float dd = g0 * da;
      if constexpr (kRS) {
        const int hs = rshift[row];
        const float ddr = ldexpf(dd, -hs);
        if (__builtin_amdgcn_ballot_w64(!foldable(ddr, dd)) == 0) {
#pragma unroll
          for (int f = 0; f < NF; ++f)
            v[f] = pack4(acc[i][f][0] * ddr, acc[i][f][1] * ddr, acc[i][f][2] * ddr, acc[i][f][3] * ddr);
        } else {
#pragma unroll
          for (int f = 0; f < NF; ++f)
            v[f] = pack4(ldexpf(acc[i][f][0] * dd, -hs), ldexpf(acc[i][f][1] * dd, -hs),
                         ldexpf(acc[i][f][2] * dd, -hs), ldexpf(acc[i][f][3] * dd, -hs));
        }
      } else {
#pragma unroll
        for (int f = 0; f < NF; ++f)
          v[f] = pack4(acc[i][f][0] * dd, acc[i][f][1] * dd, acc[i][f][2] * dd, acc[i][f][3] * dd);
      }
    }
#pragma unroll
    for (int f = 0; f + 1 < NF; f += 2) {
      const auto lo = __builtin_amdgcn_permlane16_swap(v[f].x, v[f + 1].x, false, false);
      const auto hi = __builtin_amdgcn_permlane16_swap(v[f].y, v[f + 1].y, false, false);
      if (valid) *reinterpret_cast<uint4*>(dst(i, row, colw + 16 * f + pc)) = uint4{lo[0], hi[0], lo[1], hi[1]};
    }
    if (NF % 2 && valid) *reinterpret_cast<uint2*>(dst(i, row, colw + 16 * (NF - 1) + 4 * q)) = v[NF - 1];
  }
}

template <int MI, int NB, bool GATE_UP, int BN, int COLS_PER_WAVE, bool GSCALE, class P, int RBE = MI>
__device__ __forceinline__ void epilogue(const P& p, const GemmBank& bank, const TileInfo& ti, int ntile,
                                         const f32x4 (&acc)[MI][NB], int mtile = 0,
                                         std::nullptr_t rshift = nullptr, IntC<RBE> = {}) {
  const float* gs = GSCALE ? bank.gs + (size_t)ti.group * bank.gs_per_expert : nullptr;
  epilogue_at<MI, NB, GATE_UP, BN, COLS_PER_WAVE>(p, gs ? gs[0] : 1.f, (GATE_UP && gs) ? gs[1] : 1.f, ti, ntile, acc,
                                                  mtile, rshift, IntC<RBE>{}, (int)(threadIdx.x & 63),
                                                  (int)(threadIdx.x >> 6));
}

}  // namespace
}  // namespace moe
