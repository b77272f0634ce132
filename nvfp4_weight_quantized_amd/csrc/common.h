// Internal declarations shared by the HIP sources of libmoe_nvfp4 (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <algorithm>

#include "../../include/moe_nvfp4.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// Two values to bf16 (round to nearest even) in one dword, lo in the low half: one
// v_cvt_pk_bf16_f32 with both operands, the same rounding as f32_to_bf16 of each.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// 16 bytes per lane from global memory straight to LDS (global_load_lds_dwordx4): lane i's bytes
// land at lds_addr + 16*i.  The global address is a wave-uniform base plus a 32-bit per-lane byte
// offset; lds_addr must be wave-uniform (it is passed in M0).  Issued from inline assembly, so the
// compiler does not count it among its outstanding loads and never waits for it: completion is the
// caller's explicit vmcnt wait, then a barrier before other waves read the data.
__device__ __forceinline__ void direct_load16(const void* base, uint32_t offset, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(offset), "s"(base), "{m0}"(lds_addr) : "memory");
}

// 4 bytes per lane from global memory straight to LDS (global_load_lds_dword): lane i's dword lands
// at lds_addr + 4*i; otherwise as direct_load16.
__device__ __forceinline__ void direct_load4(const void* base, uint32_t offset, uint32_t lds_addr) {
  asm volatile("global_load_lds_dword %0, %1" : : "v"(offset), "s"(base), "{m0}"(lds_addr) : "memory");
}

// Host-side launch helpers -----------------------------------------------------------------

// Status of the last launch on this thread; MOE_ERR_HIP if the launch was rejected.
inline moe_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// Permute -----------------------------------------------------------------------------------
constexpr int kPermuteChunk = 2048;     // slots per workgroup of the multi-block path
constexpr int kPermuteThreads = 512;    // 8 waves

inline int permute_blocks(int64_t slots) { return (int)((slots + kPermuteChunk - 1) / kPermuteChunk); }

moe_status_t launch_permute(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
                            int32_t* offsets, int32_t* sorted_slot, int32_t* slot_to_row,
                            int32_t* block_hist, hipStream_t stream);

// S2 + S3 in one workgroup for T*k <= kPermuteChunk.
moe_status_t launch_topk_permute_small(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, float* w,
                                       int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                                       int32_t* slot_to_row, hipStream_t stream);

// Route -------------------------------------------------------------------------------------
// T <= kRouterSmallTokens runs the one-pass few-token kernel, larger T the MFMA kernel; either
// also clears `zero` [n_zero] (counters of the kernels that follow in the same stream).
constexpr int kRouterSmallTokens = 32;
// partial, splits (MFMA kernel only): the K range of each tile cut into `splits` runs on as many
// workgroups; run 0 writes logits and run s partial + (s - 1) * T * E, all without the bias, and
// launch_topk_sum adds them (splits = 1: one run, bias included, partial unused).
moe_status_t launch_router_logits(const uint16_t* x, const uint16_t* w_router, const float* bias, int32_t T,
                                  int32_t H, int32_t E, float* logits, hipStream_t stream, int32_t* zero = nullptr,
                                  int32_t n_zero = 0, float* partial = nullptr, int32_t splits = 1);
// The forward's split count for the router GEMM (1 when it takes the few-token kernel or the
// one-workgroup top-k + permutation, or when its tiles alone fill the GPU).
int router_k_splits(int32_t T, int32_t H, int32_t E, int32_t k);
// Top-k after a split router: logits = (partial sums in split order) + bias, written back, then the
// selection of launch_route.
moe_status_t launch_topk_sum(float* logits, const float* partial, int32_t splits, const float* bias, int32_t T,
                             int32_t E, int32_t k, int32_t* ids, float* w, hipStream_t stream);
moe_status_t launch_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int32_t T,
                          int32_t H, int32_t E, int32_t k, bool logits_given, float* logits,
                          int32_t* ids, float* w, hipStream_t stream);

// Grouped GEMM ------------------------------------------------------------------------------
struct GemmBank {
  const uint8_t* w;      // packed nibbles, [E][Nrows][K/2] bytes in the MFMA tile layout (layout.hip)
  const uint8_t* ws;     // block scales in the tile layout: E4M3 [E][Nrows][K/16] (NVFP4) or
                         // E8M0 [E][Nrows][K/32] (MXFP4)
  const float* gs;       // dequant global scales, [E][gs_per_expert] (NVFP4; unused for MXFP4)
  int32_t gs_per_expert; // 2 (gate, up) or 1 (down)
  int32_t format;        // MOE_WEIGHT_NVFP4 or MOE_WEIGHT_MXFP4
};

struct GemmProblem {
  int32_t stage;          // MOE_GEMM_GATE_UP or MOE_GEMM_DOWN
  int32_t N;              // output columns (I for gate/up, H for down)
  int32_t K;              // reduction length (H for gate/up, I for down)
  // main bank: groups from device offsets
  GemmBank bank;
  const int32_t* offsets; // [G+1]
  int32_t G;              // number of groups
  int32_t M;              // rows of the main bank == offsets[G]
  const uint16_t* a;      // A rows source (K columns)
  const int32_t* row_index;  // NULL: identity
  int32_t row_divisor;
  uint16_t* out;          // [M (+ M_extra)][N]
  // optional extra single-expert group (the shared expert): rows [0, M_extra) read a_extra[r]
  // and write out[M + r]
  int32_t has_extra;
  GemmBank extra;
  int32_t M_extra;
  const uint16_t* a_extra;
  // Tall-tile path only: activations in the fragment-tiled layout.  Tile m of the problem's
  // 128-row m-tiles (numbered as find_tile does: the extra group's first, then the groups in
  // order) holds, for each
  // 128-column chunk c of the K dimension, 32 fragments of 1 KB: fragment F = 4*i + j holds at
  // byte 16*l (l = 16*q + n) row 16*i + n, columns [128*c + 32*j + 8*q, +8) of the tile, i.e.
  // byte offset ((m * (K/128) + c) * 32 + F) * 1024 + 16 * l.  Rows past a group's end are
  // undefined.
  int32_t a_tiled;        // 1: `a` (and the extra group's rows) are read in that layout
  uint16_t* out_tiled;    // gate/up: write h in that layout (K = N columns) instead of `out`
  // NVFP4 weights, eight-wave 128-row path only (ignored elsewhere): fp16 operand rows.
  //  Gate/up: the token rows as fp16, a16[t] = a[t] * 2^xs exactly with xs = (int16_t)row_shift[t]
  //  (launch_act_to_f16), for both `a` and `a_extra` (the same token matrix).
  //  Down (h16 set): a16 is h in the tiled layout as the gate/up launch with h16 wrote it, and
  //  row_shift[r] the power of two of h row r (the row numbering of `out`: the groups' rows, then
  //  the extra group's).
  const uint16_t* a16;
  const int32_t* row_shift;
  // h as fp16 (eight-wave 128-row path on fp16 rows, tiled output): gate/up writes each h row as
  // fp16(bf16(h) * 2^hs) with hs = row_shift[t] >> 16 of the row's token (chosen by
  // launch_act_to_f16 from a bound on |h|, exact for every element within 2^31 of the bound), and
  // the column tile 0 workgroups store hs in hshift_out[row]; down takes such h (a16, row_shift
  // above) and scales its sums back by 2^-hs.
  int32_t h16;
  int32_t* hshift_out;
  // W4A4 on NVFP4 activations: the dequant global scale of the activation rows, which then hold
  // the exact values e2m1(code) * e4m3(block scale) (launch_quantize_act_nv); the epilogue scales
  // the sums by it and the weight's global scale (alpha = 1 / (input_global_scale *
  // weight_global_scale) in the guide's section 6.1).  0: the rows are plain bf16 activations
  // (W4A16) and nothing is applied.
  float a_gscale;
  // Eight-wave 128-row path only (ignored elsewhere): kTileCounterWords words, zero on entry, from which the
  // workgroups draw their tiles after the first (one counter per XCD's share of the tile list).
  // NULL: each workgroup takes a fixed share of the tiles.
  int32_t* tile_ctr;
};
constexpr int kTileCounterWords = 8;   // words of GemmProblem::tile_ctr

// The activation global scale the epilogues apply (1 for W4A16 problems).
__host__ __device__ inline float act_gscale(const GemmProblem& p) { return p.a_gscale != 0.f ? p.a_gscale : 1.f; }

// Bound on the number of 128-row m-tiles of a problem (every non-empty group adds at most one
// partial tile), the size of the tiled layouts above.
inline long long tall_mtiles_bound(const GemmProblem& p) {
  return (p.G > 0 ? (long long)std::min(p.G, p.M) + p.M / 128 : 0LL) + (p.has_extra ? (p.M_extra + 127) / 128 : 0);
}

// True if launch_grouped_gemm runs this problem with 128-row tiles (the only path that reads or
// writes the tiled layouts).
bool grouped_gemm_uses_tall_tiles(const GemmProblem& p);

// True if launch_grouped_gemm runs this problem on the skinny (8-row) tiles.
bool grouped_gemm_uses_skinny_tiles(const GemmProblem& p);

moe_status_t launch_grouped_gemm(const GemmProblem& p, hipStream_t stream);
// x16[t][h] = fp16(x[t][h] * 2^xs) with xs = 14 - floor(log2(max_h |x[t][h]|)) (0 for a row of
// zeros or with a non-finite value): exact for every element within 2^31 of its row's largest
// magnitude.  shift[t] = (xs & 0xFFFF) | (hs << 16), where hs is the power of two of the row's h
// in the fp16 h path: with ng, nu bounds on the Euclidean norms of every gate and up weight row
// (dequantized, global scale included; 0: no fp16 h, hs = 0), |g| <= ||x|| ng and |u| <= ||x|| nu,
// so |h| = |silu(g) u| <= |g| |u| <= ||x||^2 ng nu < 2^e, and hs = 13 - e puts every h of the
// token below 2^13 (a binade of margin for the rounding of the sums and of h).  One workgroup per
// row.
moe_status_t launch_act_to_f16(const uint16_t* x, int32_t T, int32_t H, uint16_t* x16, int32_t* shift, float ng,
                               float nu, hipStream_t stream);
// True if launch_grouped_gemm would read p.a16 / p.row_shift for this problem (the gate/up one, or
// the down one when it reads fp16 h).
bool grouped_gemm_takes_f16_rows(const GemmProblem& p);

// W4A4 grouped GEMM: MXFP4 weights in the W4A4 tile layout (layout.hip) times MXFP4 activations,
// on the scaled FP4 matrix cores.  Same grouping and output as GemmProblem; the activations are
// E2M1 codes [rows][K/2] and E8M0 scales [rows][K/32] (row-major, as quantize.hip writes them).
struct GemmProblemA4 {
  int32_t stage;
  int32_t N;
  int32_t K;
  GemmBank bank;          // format MXFP4, w / ws in the W4A4 tile layout
  const int32_t* offsets;
  int32_t G;
  int32_t M;
  const uint8_t* a;       // activation codes
  const uint8_t* a_scale; // activation block scales
  const int32_t* row_index;
  int32_t row_divisor;
  uint16_t* out;
  int32_t has_extra;
  GemmBank extra;
  int32_t M_extra;
  const uint8_t* a_extra;
  const uint8_t* a_extra_scale;
  uint16_t* out_tiled;    // always NULL here (the shared epilogue's tiled-h output is W4A16 only)
};

moe_status_t launch_grouped_gemm_a4(const GemmProblemA4& p, hipStream_t stream);

// Fused decode path --------------------------------------------------------------------------
// S2..S6 of a few-token forward in one launch (micro.hip): top-k + permutation, gate/up, down and
// combine on the skinny tiles, handed from workgroup to workgroup through counters in the
// workspace that the router launch of the same forward clears.
struct FusedDecodeProblem {
  GemmProblem gu;          // gate/up: routed bank (+ shared expert as the extra group), h row-major
  GemmProblem dn;          // down: y row-major, the shared rows after the routed ones
  const float* logits;     // [T][E], from the router launch
  int32_t T, E, k, H;
  int32_t* ids;            // [T][k]
  float* w;                // [T][k]
  int32_t* counts;         // [E]
  int32_t* offsets;        // [E + 1] (also gu.offsets / dn.offsets)
  int32_t* sorted_slot;    // [T*k]   (also gu.row_index)
  int32_t* slot_to_row;    // [T*k]
  uint16_t* out;           // [T][H]
  int32_t* ctr;            // fused_decode_counter_words(...) words, zero on entry
};
constexpr int kFusedDecodeMaxTokens = 32;
constexpr int kFusedDecodeMaxSlots = 256;
constexpr int kFusedDecodeMaxExperts = 320;
// Words of the counter block (ticket, flags, one counter per m-tile).
int fused_decode_counter_words(int32_t T, int32_t k, int32_t E, bool shared);
// True if the fused launch can run this forward (few tokens, NVFP4, skinny tiles for both GEMMs).
bool fused_decode_applies(const GemmProblem& gu, int32_t T, int32_t k);
moe_status_t launch_fused_decode(const FusedDecodeProblem& p, hipStream_t stream);

// Combine -----------------------------------------------------------------------------------
moe_status_t launch_combine(const uint16_t* y_rows, const int32_t* slot_to_row, const float* w,
                            const uint16_t* y_shared, int32_t T, int32_t k, int32_t H, uint16_t* out,
                            hipStream_t stream);

// Weight tile layout ------------------------------------------------------------------------
moe_status_t launch_pack_tiles(const uint8_t* packed, const uint8_t* scales, int32_t num_tensors, int32_t rows,
                               int32_t cols, uint8_t* tiled, uint8_t* tiled_scales, hipStream_t stream);
moe_status_t launch_pack_tiles_mx(const uint8_t* packed, const uint8_t* scales, int32_t num_tensors, int32_t rows,
                                  int32_t cols, uint8_t* tiled, uint8_t* tiled_scales, hipStream_t stream);
moe_status_t launch_pack_tiles_a4(const uint8_t* packed, const uint8_t* scales, int32_t num_tensors, int32_t rows,
                                  int32_t cols, uint8_t* tiled, uint8_t* tiled_scales, hipStream_t stream);

// Quantize ----------------------------------------------------------------------------------
// Largest Euclidean norm of the dequantized gate rows / up rows of a tiled NVFP4 w13 bank (E
// experts, global scales gs [E][2]), each rounded up to fp32 and folded into bound[0] / bound[1]
// by a maximum (bound: device, two floats).
moe_status_t launch_h16_bound(const uint8_t* w13, const uint8_t* s13, const float* gs, int32_t E, int32_t I,
                              int32_t H, float* bound, hipStream_t stream);
moe_status_t launch_quantize(const float* w, int32_t num_tensors, int32_t rows, int32_t cols,
                             const float* gscale, uint8_t* packed, uint8_t* scales, hipStream_t stream);
moe_status_t launch_quantize_mx(const float* w, int32_t num_tensors, int32_t rows, int32_t cols, uint8_t* packed,
                                uint8_t* scales, hipStream_t stream);
moe_status_t launch_quantize_act_mx(const uint16_t* a, int64_t rows, int32_t cols, uint8_t* packed, uint8_t* scales,
                                    hipStream_t stream);
// NVFP4 activation rows (dequant global scale d); packed, scales and values each optional, values
// may alias a.
moe_status_t launch_quantize_act_nv(const uint16_t* a, int64_t rows, int32_t cols, float d, uint8_t* packed,
                                    uint8_t* scales, uint16_t* values, hipStream_t stream);

}  // namespace moe
