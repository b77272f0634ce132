// Grouped NVFP4 (or MXFP4) x bf16 GEMMs of the MoE layer (S4 gate/up with SiLU(gate)*up, S5
// down), gfx950.
//
// Method: weight-only W4A16 -- 16-bit activations times 4-bit weights that are dequantized to
// 16-bit inside the GEMM ("vLLM on the NVIDIA DGX Spark: A Complete Technical Guide", section 5,
// Marlin), on the NVFP4 format of section 6.1 (E2M1 pairs per byte, one E4M3 scale per 16
// elements along K, one fp32 global scale per tensor) or the MXFP4 format of section 6.4 (one
// E8M0 scale per 32 elements, no global scale; see WFmt below).  SiLU(gate)*up between the GEMMs
// as in the fused MoE of section 4.  The notes below describe NVFP4.
//
// CDNA4 design:
//  * Weights are read in the MFMA tile layout (see layout.hip): one 16-row x 128-K tile is 1 KB of
//    nibbles in lane order plus 128 B of scales, so every weight load of a wave is one contiguous
//    1 KB request.  Lane l = 16q + n owns weight row n; word j of its 16 bytes holds the 8
//    elements K [32j + 8q, +8) of MFMA step j, and byte j of its scale dword their E4M3 scale.
//  * Those bytes are dequantized in registers straight into the bf16 MFMA operand:
//    v_cvt_scalef32_pk_f32_fp4 (scale 1) gives the E2M1 values, one fp32 multiply applies the
//    block scale and v_cvt_pk_bf16_f32 packs the result.  element * block scale has at most 6
//    significant bits, so the bf16 operand is exact.  The eight-wave gate/up kernel can take the
//    token rows as fp16 instead (each row scaled by a power of two, an exact re-encoding) and
//    then builds fp16 weight operands with one packed fp16 multiply per two elements; it can also
//    write h as fp16 (each token's h rows scaled by a power of two from a bound on |h|), which the
//    eight-wave down kernel then multiplies in fp16 as well.
//  * The weights are the MFMA's first operand and the activations its second, so the 16x16
//    accumulator block is (weight row, token row): lane l = 16q + n holds token row n and four
//    consecutive output columns 4q..4q+3, stored as one 8-byte write.
//  * A (activation rows, bf16) is gathered row by row through the sorted slot list straight from
//    the token matrix -- no permuted copy -- and staged in LDS per K chunk.
//  * fp32 accumulation; the per-tensor global scales multiply the accumulators in the epilogue;
//    gate/up workgroups hold matching gate and up columns so h = silu(g)*u is formed in registers.
//  * Groups (experts) are found on the device from the offsets array: no host synchronisation.
//    Workgroups beyond the real tile count exit at once; empty experts cost nothing.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "gemm_skinny.h"
#include "gemm_tiles.h"

namespace moe {
namespace {

constexpr int kThreads = kSkinnyThreads;   // 4 waves

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

// Weight operand of MFMA step j (0..3) of one 128-K tile: word j of the lane's 16 nibble bytes
// times byte j of its scale dword.
__device__ __forceinline__ bf16x8 w_operand(const uint4& w, uint32_t sc, int j) {
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
  return dequant8(words[j], e4m3_byte(sc, j));
}

// acc[weight row][token row] += W(16x32) . X(16x32)^T
__device__ __forceinline__ f32x4 mfma(const bf16x8& w, const bf16x8& x, const f32x4& acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, x, acc, 0, 0, 0);
}

// fp16 operands (NVFP4 on fp16 token rows or fp16 h; see grouped_gemm_tall_lds_kernel).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma(const f16x8& w, const f16x8& x, const f32x4& acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(w, x, acc, 0, 0, 0);
}
// Weight operand of MFMA step j as fp16: the E2M1 values (v_cvt_scalef32_pk_f16_fp4, scale 1) times
// the E4M3 block scale as an fp16 pair (v_cvt_scalef32_pk_f16_fp8 converts two scale bytes at
// once), one packed fp16 multiply per two elements.  Exact: every E4M3 value is an fp16 value, and
// element * scale has at most 6 significant bits, lies within 6 * 448 and is a multiple of 2^-12.
__device__ __forceinline__ f16x8 w_operand16(const uint4& w, uint32_t sc, int j) {
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
  const f16x2 sp = j >= 2 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, true)
                          : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, false);
  const _Float16 s1 = (j & 1) ? sp[1] : sp[0];
  const f16x2 ss = {s1, s1};
  const uint32_t q = words[j];
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0) * ss;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1) * ss;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2) * ss;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3) * ss;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Weight formats.  NVFP4: E4M3 scale per 16 elements (128 scale bytes per tile) and fp32 global
// scales applied in the epilogue.  MXFP4 ("vLLM on the NVIDIA DGX Spark", section 6.4): one E8M0
// exponent-only scale per 32 elements -- exactly one per MFMA step -- so a tile has 64 scale bytes
// (the dword at 4*(row in tile) holds step j's scale in byte j), there is no global scale, and the
// conversion applies the scale itself: given the E8M0 byte as an fp32 exponent field,
// v_cvt_scalef32_pk_bf16_fp4 multiplies by exactly 2^(byte - 127) (byte 0 included; checked on the
// GPU), one instruction per two codes.
constexpr int kFmtNvfp4 = MOE_WEIGHT_NVFP4;
constexpr int kFmtMxfp4 = MOE_WEIGHT_MXFP4;

template <int FMT>
struct WFmt;

template <>
struct WFmt<kFmtNvfp4> {
  static constexpr int kTileScaleBytes = 128;
  static constexpr int kScaleGroup = 16;
  static constexpr bool kGlobalScale = true;
  __device__ static int s_lane(int lane) { return s_lane_offset(lane); }
  __device__ static bf16x8 operand(const uint4& w, uint32_t sc, int j) { return w_operand(w, sc, j); }
};

template <>
struct WFmt<kFmtMxfp4> {
  static constexpr int kTileScaleBytes = 64;
  static constexpr int kScaleGroup = 32;
  static constexpr bool kGlobalScale = false;
  __device__ static int s_lane(int lane) { return 4 * (lane & 15); }
  __device__ static bf16x8 operand(const uint4& w, uint32_t sc, int j) {
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
    const float scale = __uint_as_float(((sc >> (8 * j)) & 0xFFu) << 23);
    const uint32_t q = words[j];
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 3);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
};

// Skinny tiles (gemm_skinny.h): one workgroup per (m-tile, output-column tile), n fastest.
template <int NB, int BK, bool GATE_UP>
__global__ __launch_bounds__(kSkinnyThreads) void grouped_gemm_skinny_kernel(GemmProblem p) {
  __shared__ SkinnyLds<BK> lds;
  const int NT = p.N / skinny_bn<NB, GATE_UP>();
  const int mtile = blockIdx.x / NT;
  skinny_tile<NB, BK, GATE_UP>(p, mtile, blockIdx.x - mtile * NT, lds);
}

// ------------------------------------------------------------------------------------------
// Short and medium tiles.  MI: 16-row A fragments per wave (BM = 16*MI); NB: 16-column B
// fragments per wave; BK: K chunk staged in LDS per barrier (a multiple of 128: BK/128 weight
// tiles per fragment per chunk).  A is copied global -> registers -> LDS one chunk ahead.
template <int MI, int NB, int BK, bool GATE_UP, int FMT>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmProblem p) {
  using F = WFmt<FMT>;
  constexpr int BM = 16 * MI;
  constexpr int COLS_PER_WAVE = GATE_UP ? 16 * (NB / 2) : 16 * NB;   // output columns per wave
  constexpr int BN = 4 * COLS_PER_WAVE;                               // output columns per workgroup
  constexpr int NS = BK / 128;          // weight tiles per fragment per chunk
  constexpr int A_TPR = BK / 8;         // threads per A row (16 bytes each)
  constexpr int A_RPP = kThreads / A_TPR;   // A rows per pass
  constexpr int A_ITERS = (BM + A_RPP - 1) / A_RPP;
  static_assert(BK % 128 == 0 && BK <= 512, "BK must be 128, 256 or 512");
  __shared__ __attribute__((aligned(16))) uint16_t As[A_ITERS * A_RPP][BK + kAPad];
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
  const int ktiles = K / 128;

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

  // B tiles this lane reads
  const int q = lane >> 4;
  const int nl = lane & 15;
  const size_t rows_per_expert = GATE_UP ? 2 * (size_t)p.N : (size_t)p.N;
  const uint8_t* wexp = bank.w + (size_t)ti.group * rows_per_expert * (size_t)(K / 2) + w_lane_offset(lane);
  const uint8_t* sexp = bank.ws + (size_t)ti.group * rows_per_expert * (size_t)(K / F::kScaleGroup) + F::s_lane(lane);
  const uint8_t* wptr[NB];
  const uint8_t* sptr[NB];
#pragma unroll
  for (int f = 0; f < NB; ++f) {
    const size_t t0 = (size_t)frag_row_block<NB, GATE_UP, BN, COLS_PER_WAVE>(f, ntile, wave, p.N) * ktiles;
    wptr[f] = wexp + t0 * 1024;
    sptr[f] = sexp + t0 * F::kTileScaleBytes;
  }

  f32x4 acc[MI][NB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int f = 0; f < NB; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 a_next[A_ITERS];
  uint4 b_next[NB][NS];
  uint32_t s_next[NB][NS];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it)
      a_next[it] = arow[it] ? *reinterpret_cast<const uint4*>(arow[it] + (size_t)c * BK + acol) : uint4{0, 0, 0, 0};
#pragma unroll
    for (int f = 0; f < NB; ++f)
#pragma unroll
      for (int v = 0; v < NS; ++v) {
        const size_t t = (size_t)c * NS + v;
        b_next[f][v] = load_stream16(wptr[f] + t * 1024);
        s_next[f][v] = load_stream4(sptr[f] + t * F::kTileScaleBytes);
      }
  };
  load_chunk(0);

  for (int c = 0; c < nK; ++c) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it)
      *reinterpret_cast<uint4*>(&As[tid / A_TPR + A_RPP * it][acol]) = a_next[it];
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
        bf16x8 wfrag[NB];
#pragma unroll
        for (int f = 0; f < NB; ++f) wfrag[f] = F::operand(bq[f][v], sc[f][v], j);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const bf16x8 xfrag = *reinterpret_cast<const bf16x8*>(&As[16 * i + nl][128 * v + 32 * j + 8 * q]);
#pragma unroll
          for (int f = 0; f < NB; ++f) acc[i][f] = mfma(wfrag[f], xfrag, acc[i][f]);
        }
      }
  }
  epilogue<MI, NB, GATE_UP, BN, COLS_PER_WAVE, WFmt<FMT>::kGlobalScale>(p, bank, ti, ntile, acc);
}

// ------------------------------------------------------------------------------------------
// Tall tiles (many rows per expert): 128-row workgroup tiles, K chunk 128.
//  * A chunks go global -> LDS directly (global_load_lds_dwordx4, 16 bytes per lane; lane i of a
//    wave lands at LDS address M0 + 16*i), triple-buffered with eight waves (two chunks in
//    flight) and double-buffered with four, one barrier per chunk.  A chunk is
//    stored as 32 MFMA fragments of 1 KB: fragment (i, j) holds, at 16*l for lane l = 16q + n, row
//    16i + n and K [32j + 8q, +8) of the chunk.  Every fragment read is then one contiguous 1 KB
//    ds_read_b128 (free of bank conflicts), and every direct load reads 64 contiguous bytes from
//    each of 16 rows.
//  * The direct loads are issued from inline assembly and waited for explicitly (an s_waitcnt
//    vmcnt and a barrier at the end of each chunk).  Issued through the compiler builtin, the
//    compiler cannot tell that the loads in flight into one buffer leave the others alone and
//    drains them before every LDS read, which serialises loading and computing.
//  * B tiles in registers, prefetched one chunk ahead; the end-of-chunk wait names the prefetch
//    registers, so the compiler waits for them there and nowhere earlier.  Within a chunk the
//    next MFMA step's weight operands are dequantized while the current step's MFMAs run.
//  * The number of 16-row blocks holding real rows is a template parameter of the main loop (one
//    instantiation per count): blocks past the group's last row cost nothing and the loop body
//    has no per-block branches.
//  * Tile order is XCD-aware: workgroup b runs on XCD b % 8; each XCD walks a contiguous range of
//    (m-tile, n-tile) pairs, n fastest, so the A rows of an m-tile are reused from that XCD's L2.
//  * Launched with WAVES = 4 (two workgroups per CU, two waves per SIMD, at most 256 registers per
//    lane) for down GEMMs whose width is not a multiple of 512 and gate/up outputs whose width is
//    not a multiple of 256; the rest takes the eight-wave kernel below (one workgroup per CU).  The
//    WAVES = 8 form of this kernel (three A buffers) is kept compilable but not launched.
constexpr int kTallBK = 128;
constexpr int kTallRows = 128;
// groups the eight-wave kernel keeps in LDS (its tile list)
constexpr int kTallMaxGroups = 1024;

template <int NB, bool GATE_UP, int WAVES, int FMT>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void grouped_gemm_tall_kernel(GemmProblem p) {
  using F = WFmt<FMT>;
  constexpr int MI = kTallRows / 16;
  constexpr int BM = kTallRows;
  constexpr int BK = kTallBK;
  constexpr int STEPS = BK / 32;                       // MFMA k-steps per chunk
  constexpr int COLS_PER_WAVE = GATE_UP ? 16 * (NB / 2) : 16 * NB;
  constexpr int BN = WAVES * COLS_PER_WAVE;
  constexpr int FRAGS = MI * STEPS;                    // 1 KB A fragments per chunk
  constexpr int BUF_BYTES = FRAGS * 1024;              // 32 KB
  constexpr int A_ITERS = FRAGS / WAVES;               // fragments (direct loads) per wave per chunk
  static_assert(STEPS == 4 && FRAGS % WAVES == 0, "chunk layout");
  constexpr int NBUF = WAVES == 8 ? 3 : 2;              // A chunk buffers (LDS: 96 or 64 KB)
  constexpr int AHEAD = NBUF - 1;                       // A chunks in flight beyond the current one
  __shared__ __attribute__((aligned(1024))) uint8_t As[NBUF * BUF_BYTES];
  __shared__ uint32_t s_aoff[BM];
  __shared__ TileInfo tile;
  __shared__ int tile_ok;
  __shared__ int tile_n;
  __shared__ int tile_m;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4;
  const int nl = lane & 15;
  const int NT = p.N / BN;

  if (wave == 0) {
    const int total = count_tiles<BM>(p) * NT;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    const int L = (blockIdx.x % kXcds) * per_xcd + slot;
    bool ok = slot < per_xcd && L < total;
    if (ok) ok = find_tile<BM>(p, L / NT, &tile);
    if (lane == 0) {
      tile_ok = ok ? 1 : 0;
      tile_n = ok ? L % NT : 0;
      tile_m = ok ? L / NT : 0;
    }
  }
  __syncthreads();
  if (!tile_ok) return;
  TileInfo ti;   // wave-uniform copies (scalar registers)
  ti.group = __builtin_amdgcn_readfirstlane(tile.group);
  ti.row0 = __builtin_amdgcn_readfirstlane(tile.row0);
  ti.rows = __builtin_amdgcn_readfirstlane(tile.rows);
  ti.a_row0 = __builtin_amdgcn_readfirstlane(tile.a_row0);
  ti.extra = __builtin_amdgcn_readfirstlane(tile.extra);
  const int ntile = __builtin_amdgcn_readfirstlane(tile_n);
  const int mtile = __builtin_amdgcn_readfirstlane(tile_m);
  const GemmBank& bank = ti.extra ? p.extra : p.bank;
  const int K = p.K;
  const int nK = K / BK;

  // A rows: byte offset of each of the tile's rows (rows past the group repeat a valid row).
  // Tiled A: the tile's chunks are contiguous 32 KB blocks already in fragment order.
  const uint8_t* abase = reinterpret_cast<const uint8_t*>(p.a_tiled ? p.a : (ti.extra ? p.a_extra : p.a));
  if (p.a_tiled) abase += (size_t)mtile * nK * BUF_BYTES;
  if (tid < BM && !p.a_tiled) {
    const int R = ti.a_row0 + min(tid, ti.rows - 1);
    const int src = (!ti.extra && p.row_index) ? p.row_index[R] / p.row_divisor : R;
    s_aoff[tid] = (uint32_t)src * (uint32_t)K * 2u;
  }
  __syncthreads();
  // Direct load `it` of wave `wave` fills fragment F = wave + WAVES*it = (i = F/4, j = F%4): this
  // lane fetches row 16*i + nl at chunk column 32*j + 8*q (byte offsets from the chunk's first column).
  uint32_t aoff[A_ITERS];
#pragma unroll
  for (int it = 0; it < A_ITERS; ++it) {
    const int F = wave + WAVES * it;
    aoff[it] = p.a_tiled ? (uint32_t)(F * 1024 + 16 * lane)
                         : s_aoff[16 * (F >> 2) + nl] + (uint32_t)(64 * (F & 3) + 16 * q);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)As;

  // B tiles of this wave: wave-uniform tile bases plus a per-lane offset
  const int ktiles = K / 128;
  const size_t rows_per_expert = GATE_UP ? 2 * (size_t)p.N : (size_t)p.N;
  const uint8_t* wexp = bank.w + (size_t)ti.group * rows_per_expert * (size_t)(K / 2);
  const uint8_t* sexp = bank.ws + (size_t)ti.group * rows_per_expert * (size_t)(K / F::kScaleGroup);
  const uint32_t w_lane = (uint32_t)w_lane_offset(lane);
  const uint32_t s_lane = (uint32_t)F::s_lane(lane);
  uint32_t tile0[NB];
#pragma unroll
  for (int f = 0; f < NB; ++f)
    tile0[f] = (uint32_t)(frag_row_block<NB, GATE_UP, BN, COLS_PER_WAVE>(f, ntile, wave, p.N) * ktiles);

  f32x4 acc[MI][NB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int f = 0; f < NB; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 bn[NB];
  uint32_t sn[NB];
  auto load_b = [&](int c) {
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      const size_t t = (size_t)tile0[f] + (size_t)c;
      bn[f] = *reinterpret_cast<const uint4*>(wexp + t * 1024 + w_lane);
      sn[f] = *reinterpret_cast<const uint32_t*>(sexp + t * F::kTileScaleBytes + s_lane);
    }
  };
  auto issue_a = [&](int c, int buf) {
    const uint8_t* src = abase + (size_t)c * (p.a_tiled ? BUF_BYTES : BK * 2);
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it)
      direct_load16(src, aoff[it], lds0 + (uint32_t)(buf * BUF_BYTES + (wave + WAVES * it) * 1024));
  };
  // Every load of the chunk in flight (direct A loads and the B prefetch) has landed; the B
  // registers are operands so that the compiler places its own wait for them here.
  auto wait_chunk = [&]() {
#pragma unroll
    for (int f = 0; f < NB; ++f)
      asm volatile("s_waitcnt vmcnt(0)" : "+v"(bn[f].x), "+v"(bn[f].y), "+v"(bn[f].z), "+v"(bn[f].w), "+v"(sn[f])
                   :
                   : "memory");
  };
  // The main loop, for RB 16-row blocks of real rows.
  // Every load but this wave's last A_ITERS (the A chunk two ahead, issued last) has landed.
  auto wait_keep_a = [&]() {
    static_assert(AHEAD == 1 || A_ITERS == 4, "the vmcnt literal below counts one chunk's direct loads");
#pragma unroll
    for (int f = 0; f < NB; ++f)
      asm volatile("s_waitcnt vmcnt(4)" : "+v"(bn[f].x), "+v"(bn[f].y), "+v"(bn[f].z), "+v"(bn[f].w), "+v"(sn[f])
                   :
                   : "memory");
  };
  // The main loop, for RB 16-row blocks of real rows.  Per chunk c: the B prefetch of c + 1 is
  // issued, then the A direct loads of c + AHEAD; at the end of the chunk everything but the
  // newest A loads must have landed (the A chunk c + 1 and B c + 1 are then ready).
  auto run = [&](auto rb_const) {
    constexpr int RB = decltype(rb_const)::value;
    issue_a(0, 0);
    load_b(0);
    if (AHEAD == 2 && nK > 1) {
      issue_a(1, 1);
      wait_keep_a();
    } else {
      wait_chunk();
    }
    __syncthreads();
    for (int c = 0; c < nK; ++c) {
      uint4 bq[NB];
      uint32_t sc[NB];
#pragma unroll
      for (int f = 0; f < NB; ++f) {
        bq[f] = bn[f];
        sc[f] = sn[f];
      }
      if (c + 1 < nK) load_b(c + 1);
      if (c + AHEAD < nK) issue_a(c + AHEAD, (c + AHEAD) % NBUF);
      const uint8_t* abuf = As + (c % NBUF) * BUF_BYTES + 16 * lane;
      auto frag = [&](int j, int i) { return *reinterpret_cast<const bf16x8*>(abuf + (STEPS * i + j) * 1024); };
      // The next step's weight operands are dequantized while this step's MFMAs run, and each
      // activation fragment is read D row blocks before its MFMAs (within the chunk: the next
      // chunk's buffer is complete only after the barrier that ends this one).  Instruction order
      // per row block: one LDS read, then NB times an MFMA and up to VPM VALU instructions.
      constexpr int D = RB < 2 ? RB : 2;
      constexpr int VPM = (NB * (FMT == kFmtMxfp4 ? 11 : 33) / 2 + NB * RB - 1) / (NB * RB);
      bf16x8 wcur[NB];
#pragma unroll
      for (int f = 0; f < NB; ++f) wcur[f] = F::operand(bq[f], sc[f], 0);
      bf16x8 xs[D];
#pragma unroll
      for (int d = 0; d < D; ++d) xs[d] = frag(0, d);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < STEPS; ++j) {
        bf16x8 wnext[NB];
        bf16x8 x[RB + D];
#pragma unroll
        for (int d = 0; d < D; ++d) x[d] = xs[d];
        if (j + 1 < STEPS) {
#pragma unroll
          for (int f = 0; f < NB; ++f) wnext[f] = F::operand(bq[f], sc[f], j + 1);
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          if (i + D < RB) x[i + D] = frag(j, i + D);
          else if (j + 1 < STEPS) x[i + D] = frag(j + 1, i + D - RB);
#pragma unroll
          for (int f = 0; f < NB; ++f) acc[i][f] = mfma(wcur[f], x[i], acc[i][f]);
        }
        if (j + 1 < STEPS) {
          // the dequantized operands exist inside this region (code generation may otherwise
          // compute them next to their first use, after it)
#pragma unroll
          for (int f = 0; f < NB; ++f) asm volatile("" : "+v"(wnext[f]));
#pragma unroll
          for (int b = 0; b < RB; ++b) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
            for (int m = 0; m < NB; ++m) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < STEPS) {
#pragma unroll
          for (int f = 0; f < NB; ++f) wcur[f] = wnext[f];
#pragma unroll
          for (int d = 0; d < D; ++d) xs[d] = x[RB + d];
        }
      }
      if (AHEAD == 2 && c + 2 < nK)
        wait_keep_a();
      else
        wait_chunk();
      __syncthreads();
    }
    // only the RB blocks with real rows are stored: the other accumulators are never live
    epilogue<MI, NB, GATE_UP, BN, COLS_PER_WAVE, WFmt<FMT>::kGlobalScale>(p, bank, ti, ntile, acc, mtile, nullptr,
                                                                          IntC<RB>{});
  };
  switch ((ti.rows + 15) / 16) {
    case 1: run(IntC<1>{}); break;
    case 2: run(IntC<2>{}); break;
    case 3: run(IntC<3>{}); break;
    case 4: run(IntC<4>{}); break;
    case 5: run(IntC<5>{}); break;
    case 6: run(IntC<6>{}); break;
    case 7: run(IntC<7>{}); break;
    default: run(IntC<8>{}); break;
  }
}

// ------------------------------------------------------------------------------------------
// Tall tiles with eight waves (two per SIMD, one workgroup per CU), every operand by direct loads:
// the gate/up kernel for 128-row tiles whenever the output width is a multiple of 256, and the
// down kernel when it is a multiple of 512.  Each wave holds all 128 rows of the tile and NB weight
// fragments; the workgroup covers 8 * 16 * NB weight rows.
//  * Persistent (K of six chunks or more): one workgroup per compute unit walks its tiles.  Tiles
//    come from per-XCD counters (the forward's workspace), each XCD drawing from its own window of
//    the tile list and then from the others'; without counters a workgroup takes every spx-th tile
//    of its XCD's window.  The next tile is found during the current one's first chunks (tile list
//    and group offsets in LDS), its rows gathered, and its first two chunks loaded during the
//    current one's last two, so consecutive tiles run back to back (measured: 5% off the prefill
//    gate/up time, 4% off the long prefill's, against one workgroup per tile).  Nothing crosses
//    from tile to tile in registers: the main loop's row-count variants do not share registers
//    well, and state passed between them spilled.
//  * Staging: activation chunks (32 KB, fragment order as above) by direct loads into three LDS
//    buffers, two chunks ahead; each wave's weight tiles (1 KB each) and their scale dwords (one per
//    lane) by direct loads into the wave's own LDS slot, one chunk ahead, read back into registers
//    during the last MFMA step of the chunk before the one that uses them.  No load of the main loop
//    is visible to the compiler, so the only waits are the explicit ones.  (With the weights loaded
//    into registers by ordinary loads, the compiler's own wait before their first use also drains
//    every direct load issued after them -- loads complete in order and it cannot count the direct
//    loads.)
//  * Software pipeline inside the wave: while the MFMAs of step j run, the same wave dequantizes the
//    weight operands of step j + 1, and each activation fragment is read from LDS two row blocks
//    before the MFMAs that use it.  The instruction order interleaves them (sched_group_barrier: per
//    row block one LDS read, then NB times an MFMA followed by up to VPM VALU instructions), so the
//    dequantization issues while the matrix core works instead of in a burst beside it (measured:
//    4-6% off the NVFP4 gate/up time against the same kernel with the dequantization of a step done
//    before its MFMAs, and 5% off the MXFP4 down GEMM against the four-wave kernel).
//  * Chunk c, in order: the activations of chunk c + 2 into the buffer chunk c - 1 used; MFMA steps
//    0..2; in step 3 the wait for this wave's activations and weights of chunk c + 1, the slot's read
//    into registers and the first RB - 2 row blocks of MFMAs beside the next chunk's first
//    dequantization; then the weights of chunk c + 2 into the slot and the chunk's one barrier (after
//    it every wave's share of chunk c + 1 has landed, and every read of chunk c's buffer has
//    returned), and the last two row blocks beside the reads of chunk c + 1's first fragments.
//  * The 16-row blocks of the tile beyond the group's rows are neither computed nor stored (a
//    template parameter counts the blocks with real rows; their accumulators are never live).
//  * A16: fp16 operands, NVFP4 only -- gate/up on the token rows as fp16 (launch_act_to_f16), down
//    on h as the gate/up launch wrote it in fp16.  Each tile's row powers of two enter LDS beside
//    its rows (s_shift; for the next tile by direct loads, one tile ahead) and the epilogue takes
//    them out of the sums exactly.
//  * Accumulators stay in the ordinary registers (128 per lane at NB = 4): with 512 registers for a
//    single wave per SIMD, the compiler keeps 16x16x32 accumulators in the accumulation registers but
//    does not tie each MFMA's result to its accumulator input, and copies every accumulator through
//    ordinary registers once per loop iteration (seen in the generated code of a four-wave form).
// H16 (gate/up on fp16 rows): the fp16 h epilogue (GemmProblem::h16), a variant of its own so that
// each variant's code holds one epilogue form.
template <int NB, bool GATE_UP, int FMT, bool A16, bool H16 = false>
__global__ __launch_bounds__(512, 1) void grouped_gemm_tall_lds_kernel(GemmProblem p) {
  using F = WFmt<FMT>;
  static_assert(!A16 || FMT == kFmtNvfp4, "fp16 rows: NVFP4 only");
  static_assert(!H16 || (GATE_UP && A16), "fp16 h: written by the gate/up GEMM on fp16 rows");
  using OpT = typename std::conditional<A16, f16x8, bf16x8>::type;
  auto w_op = [](const uint4& w, uint32_t sc, int j) -> OpT {
    if constexpr (A16) return w_operand16(w, sc, j);
    else return F::operand(w, sc, j);
  };
  constexpr int WAVES = 8;
  constexpr int MI = kTallRows / 16;
  constexpr int BM = kTallRows;
  constexpr int BK = kTallBK;
  constexpr int STEPS = BK / 32;
  constexpr int COLS_PER_WAVE = GATE_UP ? 16 * (NB / 2) : 16 * NB;
  constexpr int BN = WAVES * COLS_PER_WAVE;
  constexpr int FRAGS = MI * STEPS;
  constexpr int A_BYTES = FRAGS * 1024;                // 32 KB per activation chunk
  constexpr int A_ITERS = FRAGS / WAVES;               // direct loads per wave per activation chunk
  constexpr int NA = 3;                                // activation chunk buffers
  constexpr int W_WAVE = NB * (1024 + 256);            // one wave's weight slot
  constexpr int W_BYTES = WAVES * W_WAVE;
  static_assert(STEPS == 4 && FRAGS % WAVES == 0 && A_ITERS * WAVES == FRAGS, "chunk layout");
  static_assert(BM == 2 * 64, "the first two waves gather the tile's rows");
  static_assert(NA * A_BYTES + W_BYTES <= 140 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NA * A_BYTES + W_BYTES];
  __shared__ uint32_t s_aoff[BM];                      // byte offset of each A row of a tile
  __shared__ uint32_t s_ridx[BM];                      // row_index entries of the next tile's rows
  __shared__ int s_shift[2][A16 ? BM : 1];             // fp16 row shifts, per tile slot
  __shared__ int s_off[kTallMaxGroups + 1];            // group row offsets
  __shared__ int s_tstart[kTallMaxGroups + 1];         // first m-tile of each group
  __shared__ int s_tile[2][8];                         // tile slots: index (-1: none), then its Tile

  // The argument block through a pointer the optimizer cannot follow: a field read through it is a
  // scalar load from the argument segment where it is read, so the fields that only the per-tile
  // paths need hold no scalar registers through the main loop.
  auto args = []() {
    auto ptr = (const __attribute__((address_space(4))) GemmProblem*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ptr));
    return ptr;
  };
  // a pointer every lane holds alike, in scalar registers (the direct loads take their base there)
  auto uniform = [](const void* ptr) {
    const uint64_t v = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
  };

  // lane indices are taken afresh (lane_now) wherever a per-tile path needs them, so that none is
  // held in a register through the main loop
  const int tid = threadIdx.x;
  const int lane = lane_now();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nK = p.K / BK;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  const uint32_t ridx0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)s_ridx;
  const uint32_t shift0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)&s_shift[0][0];

  // The tile list: m-tiles of the extra group first, then each group's (the numbering of the tiled
  // activation layouts), p.N / BN column tiles each; tile L = m-tile * (p.N / BN) + column tile.
  if (p.G > 0)
    for (int g = tid; g <= p.G; g += 512) s_off[g] = p.offsets[g];
  __syncthreads();
  if (wave == 0) {
    int carry = p.has_extra ? (p.M_extra + BM - 1) / BM : 0;
    for (int g0 = 0; g0 < p.G; g0 += 64) {
      const int g = g0 + lane;
      const int cnt = g < p.G ? (s_off[g + 1] - s_off[g] + BM - 1) / BM : 0;
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (g < p.G) s_tstart[g] = carry + incl - cnt;
      carry += __shfl(incl, 63);
    }
    if (lane == 0) s_tstart[p.G] = carry;
  }
  __syncthreads();
  const int total = __builtin_amdgcn_readfirstlane(s_tstart[p.G]) * (p.N / BN);

  // Work split: XCD X (blockIdx % 8) owns the window [X * pxd, X * pxd + wsize(X)) of the list, so
  // the tiles that share activation rows or an expert's weights run on one L2.  Workgroup `slot`
  // of the XCD starts on tile X * pxd + slot; with counters, each further tile is a ticket drawn
  // from the window's counter (tile X * pxd + spx + ticket), and once the window is spent, from
  // the other XCDs' windows in turn; without, the workgroup takes every spx-th tile of its window.
  const int X = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int spx = gridDim.x / kXcds;
  const int pxd = (total + kXcds - 1) / kXcds;
  auto wsize = [&](int y) { return max(0, min(total, (y + 1) * pxd) - y * pxd); };
  // the next tile is found during the current one, which takes six chunks at least
  const bool chain = nK >= 6;
  const bool dyn = chain && p.tile_ctr != nullptr;
  int ywin = 0;       // wave 0: windows X .. X + ywin - 1 (mod 8) hand out no more tickets
  int tpend = 0;      // wave 0, lane 0: a ticket drawn on window X + ywin and not looked at yet
  bool pend = false;
  // wave 0: the next tile from the counters (the pending ticket first), -1 when all are spent
  auto draw = [&]() -> int {
    int32_t* const ctr = args()->tile_ctr;
#pragma nounroll
    for (; ywin < kXcds; ++ywin) {
      const int y = (X + ywin) % kXcds;
      const int n = wsize(y) - spx;
      int t;
      if (pend) {
        pend = false;
        t = __builtin_amdgcn_readfirstlane(tpend);
      } else {
        if (n <= 0) continue;
        t = 0;
        if (lane_now() == 0) t = __hip_atomic_fetch_add(ctr + y, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        t = __builtin_amdgcn_readfirstlane(t);
      }
      if (t < n) return y * pxd + spx + t;
    }
    return -1;
  };
  struct Tile {
    int L, group, row0, rows, a_row0, extra, ntile, mtile;
  };
  // wave 0: tile L of the list (-1: none) into slot sl
  auto publish = [&](int L, int sl) {
    const auto* a = args();
    Tile t{L, 0, 0, 0, 0, 0, 0, 0};
    if (L >= 0) {
      const int NT = a->N / BN;
      const int xt = a->has_extra ? (a->M_extra + BM - 1) / BM : 0;
      t.mtile = L / NT;
      t.ntile = L - t.mtile * NT;
      if (t.mtile < xt) {
        t.extra = 1;
        t.a_row0 = t.mtile * BM;
        t.row0 = a->M + t.a_row0;
        t.rows = min(BM, a->M_extra - t.a_row0);
      } else {
        // the last group whose first m-tile is at most mtile (empty groups share their start)
        int lo = 0, hi = a->G - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (__builtin_amdgcn_readfirstlane(s_tstart[mid]) <= t.mtile) lo = mid;
          else hi = mid - 1;
        }
        t.group = lo;
        t.row0 = __builtin_amdgcn_readfirstlane(s_off[lo]) +
                 (t.mtile - __builtin_amdgcn_readfirstlane(s_tstart[lo])) * BM;
        t.a_row0 = t.row0;
        t.rows = min(BM, __builtin_amdgcn_readfirstlane(s_off[lo + 1]) - t.row0);
      }
    }
    if (lane_now() == 0) {
      s_tile[sl][0] = t.L;
      s_tile[sl][1] = t.group;
      s_tile[sl][2] = t.row0;
      s_tile[sl][3] = t.rows;
      s_tile[sl][4] = t.a_row0;
      s_tile[sl][5] = t.extra;
      s_tile[sl][6] = t.ntile;
      s_tile[sl][7] = t.mtile;
    }
    return t;
  };
  // the tile in slot sl, read where needed (the address is hidden from the optimizer, which would
  // otherwise keep an earlier read of the slot in registers instead)
  auto fetch = [&](int sl) {
    const __attribute__((address_space(3))) int* v = (__attribute__((address_space(3))) int*)&s_tile[sl][0];
    asm volatile("" : "+v"(v));
    Tile t;
    t.L = __builtin_amdgcn_readfirstlane(v[0]);
    t.group = __builtin_amdgcn_readfirstlane(v[1]);
    t.row0 = __builtin_amdgcn_readfirstlane(v[2]);
    t.rows = __builtin_amdgcn_readfirstlane(v[3]);
    t.a_row0 = __builtin_amdgcn_readfirstlane(v[4]);
    t.extra = __builtin_amdgcn_readfirstlane(v[5]);
    t.ntile = __builtin_amdgcn_readfirstlane(v[6]);
    t.mtile = __builtin_amdgcn_readfirstlane(v[7]);
    return t;
  };

  if (wave == 0) publish(slot < wsize(X) ? X * pxd + slot : dyn ? draw() : -1, 0);
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(s_tile[0][0]) < 0) return;
  // the first tile's rows (ordinary loads: no direct load is in flight yet)
  {
    const Tile t = fetch(0);
    if (tid < BM && !p.a_tiled) {
      const int R = t.a_row0 + min(tid, t.rows - 1);
      const int src = (!t.extra && p.row_index) ? p.row_index[R] / p.row_divisor : R;
      s_aoff[tid] = (uint32_t)src * (uint32_t)p.K * 2u;
      if (A16) s_shift[0][tid] = p.row_shift[src];
    } else if (A16 && !GATE_UP && tid < BM) {
      // fp16 h (tiled): the power of two of each h row, in the output's row numbering
      s_shift[0][tid] = p.row_shift[t.row0 + min(tid, t.rows - 1)];
    }
  }
  __syncthreads();

  // Per-tile operand bases (uniform).
  struct Ctx {
    const uint8_t* abase;
    const uint8_t* wexp;
    const uint8_t* sexp;
    uint32_t t0[NB];
    uint32_t astride;
  };
  auto make_ctx = [&](const Tile& t) {
    const auto* a = args();
    Ctx c;
    const int K = a->K;
    const size_t rows_per_expert = GATE_UP ? 2 * (size_t)a->N : (size_t)a->N;
    const uint8_t* w = t.extra ? a->extra.w : a->bank.w;
    const uint8_t* ws = t.extra ? a->extra.ws : a->bank.ws;
    const uint16_t* ab = A16 ? a->a16 : a->a_tiled ? a->a : (t.extra ? a->a_extra : a->a);
    c.abase = reinterpret_cast<const uint8_t*>(ab);
    if (a->a_tiled) c.abase += (size_t)t.mtile * nK * A_BYTES;
    c.astride = a->a_tiled ? A_BYTES : BK * 2;
    c.wexp = w + (size_t)t.group * rows_per_expert * (size_t)(K / 2);
    c.sexp = ws + (size_t)t.group * rows_per_expert * (size_t)(K / F::kScaleGroup);
#pragma unroll
    for (int f = 0; f < NB; ++f)
      c.t0[f] = __builtin_amdgcn_readfirstlane(
          (uint32_t)(frag_row_block<NB, GATE_UP, BN, COLS_PER_WAVE>(f, t.ntile, wave, a->N) * (K / 128)));
    return c;
  };
  // direct load `it` of this wave fills fragment Fi = wave + WAVES*it: row block Fi/4, MFMA step
  // Fi%4 (row offsets from s_aoff, which holds the rows of the tile about to be loaded)
  auto row_offsets = [&](uint32_t (&ao)[A_ITERS]) {
    const bool tiled = args()->a_tiled;
    const int l = lane_now();
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it) {
      const int Fi = wave + WAVES * it;
      ao[it] = tiled ? (uint32_t)(Fi * 1024 + 16 * l)
                     : s_aoff[16 * (Fi >> 2) + (l & 15)] + (uint32_t)(64 * (Fi & 3) + 16 * (l >> 4));
    }
  };
  const uint32_t wlane = (uint32_t)w_lane_offset(lane);
  const uint32_t slane = (uint32_t)F::s_lane(lane);
  const uint32_t wslot0 = (uint32_t)(NA * A_BYTES + wave * W_WAVE);
  // this lane's bytes of the wave's weight slot: tiles at wq + 1024 f, scale dwords at wsc + 256 f
  // (two bases; read_w hides them from loop-invariant code motion, which would otherwise hoist
  // every tile's and every scale's full address into a register of its own)
  using lds_ptr = const __attribute__((address_space(3))) uint8_t*;
  lds_ptr wq = (lds_ptr)(__attribute__((address_space(3))) uint8_t*)lds + wslot0 + 16 * lane;
  lds_ptr wsc = (lds_ptr)(__attribute__((address_space(3))) uint8_t*)lds + wslot0 + NB * 1024 + 4 * lane;

  auto issue_a = [&](const Ctx& t, const uint32_t (&ao)[A_ITERS], int c, int buf) {
    const uint8_t* src = uniform(t.abase + (size_t)c * t.astride);
#pragma unroll
    for (int it = 0; it < A_ITERS; ++it)
      direct_load16(src, ao[it], lds0 + (uint32_t)(buf * A_BYTES + (wave + WAVES * it) * 1024));
  };
  auto issue_w = [&](const Ctx& t, int c) {
    const uint32_t dst = lds0 + wslot0;
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      const uint32_t tt = t.t0[f] + (uint32_t)c;
      direct_load16(uniform(t.wexp + (size_t)tt * 1024u), wlane, dst + f * 1024);
      direct_load4(uniform(t.sexp + (size_t)tt * (size_t)F::kTileScaleBytes), slane, dst + NB * 1024 + f * 256);
    }
  };
  auto wait_vm = [](auto n_const) {
    constexpr int N = decltype(n_const)::value;
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
  };
  // every LDS read this wave issued has returned (before a direct load may overwrite what it read)
  auto wait_lds_reads = []() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); };
  // this wave's weights of one chunk, from its slot to registers
  auto read_w = [&](uint4 (&bq)[NB], uint32_t (&sc)[NB]) {
    asm volatile("" : "+v"(wq), "+v"(wsc));
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
      const u32x4_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(wq + f * 1024);
      bq[f] = uint4{v.x, v.y, v.z, v.w};
      sc[f] = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(wsc + f * 256);
    }
  };
  auto frag = [&](const uint8_t* buf, int j, int i) -> OpT {
    return *reinterpret_cast<const OpT*>(buf + (STEPS * i + j) * 1024 + 16 * lane);
  };
  // The values exist at this point of the program: code generation may otherwise compute the
  // next step's weight operands next to their first use, after the step's scheduling region,
  // instead of in it between the MFMAs.
  auto pin = [](OpT (&v)[NB]) {
#pragma unroll
    for (int f = 0; f < NB; ++f) asm volatile("" : "+v"(v[f]));
  };

  int par = 0;   // tile slot (s_tile, s_shift) of the current tile
  int cb = 0;    // LDS buffer of the current tile's first chunk
  bool has_next = false;

  // First tile: its chunk 0 (weights into the slot, activations into buffer 0) landed and visible,
  // its chunk 1 activations in flight.  Every later tile starts in the same state, its first two
  // chunks loaded during the last two chunks of the tile before; no register carries over from
  // tile to tile (the row-count variants below do not share registers well).
  {
    const Ctx c0 = make_ctx(fetch(0));
    uint32_t ao[A_ITERS];
    row_offsets(ao);
    issue_w(c0, 0);
    issue_a(c0, ao, 0, 0);
    if (nK > 1) {
      issue_a(c0, ao, 1, 1);
      wait_vm(IntC<A_ITERS>{});
    } else {
      wait_vm(IntC<0>{});
    }
    __syncthreads();
  }

  // Bookkeeping of the next tile, spread over the current tile's first chunks so that each step's
  // loads are covered by a wait the main loop does anyway (none of them is visible to the
  // compiler, except the counter's atomic, whose result wave 0 reads one chunk later):
  //   chunk 0, step 3, wave 0: draw a ticket (counters);
  //   chunk 1, step 3, wave 0: the next tile into the other slot, its row_index entries into
  //   s_ridx;
  //   chunk 2, top: every wave reads whether there is one;
  //   chunk 3, top: the next tile's row offsets into s_aoff (and its fp16 row shifts, by direct
  //   loads, into the other s_shift slot);
  //   chunk nK - 2, top: its activations of chunk 0 are issued.
  auto hook_top = [&](int c) {
    if (c == 2) {
      has_next = __builtin_amdgcn_readfirstlane(s_tile[par ^ 1][0]) >= 0;
    } else if (c == 3 && has_next) {
      const auto* a = args();
      if (!a->a_tiled && wave < BM / 64) {
        const int r = wave * 64 + lane_now();
        const Tile nt = fetch(par ^ 1);
        const int R = nt.a_row0 + min(r, nt.rows - 1);
        const int src = (!nt.extra && a->row_index) ? (int)(s_ridx[r] / (uint32_t)a->row_divisor) : R;
        s_aoff[r] = (uint32_t)src * (uint32_t)a->K * 2u;
        if (A16)
          direct_load4(uniform(a->row_shift), 4u * (uint32_t)src, shift0 + (uint32_t)((par ^ 1) * BM * 4 + wave * 256));
      } else if (A16 && !GATE_UP && wave < BM / 64) {
        // fp16 h (tiled): the next tile's h-row powers of two
        const int r = wave * 64 + lane_now();
        const Tile nt = fetch(par ^ 1);
        direct_load4(uniform(a->row_shift), 4u * (uint32_t)(nt.row0 + min(r, nt.rows - 1)),
                     shift0 + (uint32_t)((par ^ 1) * BM * 4 + wave * 256));
      }
    }
  };
  auto hook_mid = [&](int c) {
    if (wave != 0) return;
    if (c == 0) {
      if (dyn && ywin < kXcds && wsize((X + ywin) % kXcds) > spx) {
        int32_t* const ctr = args()->tile_ctr;
        if (lane_now() == 0)
          tpend = __hip_atomic_fetch_add(ctr + (X + ywin) % kXcds, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        pend = true;
      }
    } else if (c == 1) {
      int Ln;
      if (dyn) {
        Ln = draw();
      } else {
        Ln = __builtin_amdgcn_readfirstlane(s_tile[par][0]) + spx;
        if (Ln - X * pxd >= wsize(X)) Ln = -1;
      }
      const Tile t = publish(Ln, par ^ 1);
      const auto* a = args();
      if (Ln >= 0 && !t.extra && a->row_index && !a->a_tiled) {
        const uint8_t* ri = uniform(a->row_index);
        const int l = lane_now();
#pragma unroll
        for (int h = 0; h < 2; ++h)
          direct_load4(ri, 4u * (uint32_t)(t.a_row0 + min(64 * h + l, t.rows - 1)), ridx0 + 256 * h);
      }
    }
  };

  // chunk modes: this tile's loads two ahead (MID), and the last two chunks, which load the next
  // tile's first two chunks if there is one (PEN, LAST)
  constexpr int MID = 0, PEN = 1, LAST = 2;

  auto run = [&](auto rb_const) {
    constexpr int RB = decltype(rb_const)::value;
    // activation fragments are read from LDS D row blocks ahead of the MFMAs that use them
    constexpr int D = RB < 2 ? RB : 2;
    // row blocks of a chunk's last step before the chunk's barrier (the next chunk's first
    // fragments are read after it)
    constexpr int H1 = RB - D;
    // VALU instructions after each MFMA: one step's dequantization (per fragment about 9.5
    // instructions on fp16 operands, 16.5 on bf16, 5.5 for MXFP4) spread over the step's MFMAs
    constexpr int VALU_STEP = NB * (A16 ? 19 : (FMT == kFmtMxfp4 ? 11 : 33)) / 2;
    constexpr int VPM = (VALU_STEP + NB * RB - 1) / (NB * RB);
    constexpr int VPM_A = H1 > 1 ? (VALU_STEP + NB * (H1 - 1) - 1) / (NB * (H1 - 1)) : VALU_STEP;
    // accumulators of the tile's row blocks (blocks past RB are never touched)
    f32x4 acc[MI][NB];
    // weight operands of the current MFMA step
    OpT wcur[NB];
    // Row blocks [I0, I1) of MFMA step j (fragments in x[i], x[0..D) read before); before block i
    // the fragment D blocks ahead is read: block i + D of this step, or past the step's end, block
    // i + D - RB of the next step (buffer nbuf, step nj) when NXT.
    auto blocks = [&](auto i0_const, auto i1_const, OpT (&x)[RB + D], const uint8_t* buf, int j, const uint8_t* nbuf,
                      int nj, auto nxt_const) {
      constexpr int I0 = decltype(i0_const)::value;
      constexpr int I1 = decltype(i1_const)::value;
      constexpr bool NXT = decltype(nxt_const)::value;
#pragma unroll
      for (int i = I0; i < I1; ++i) {
        if (i + D < RB) x[i + D] = frag(buf, j, i + D);
        else if (NXT) x[i + D] = frag(nbuf, nj, i + D - RB);
#pragma unroll
        for (int f = 0; f < NB; ++f) acc[i][f] = mfma(wcur[f], x[i], acc[i][f]);
      }
    };
    // instruction order of a region: NDS0 LDS reads first, then per row block one LDS read and
    // eight times (an MFMA, then up to V VALU instructions; none in the first block if V0 is 0)
    auto interleave = [](auto nb_const, auto nds0_const, auto v_const, auto v0_const) {
      constexpr int NBLK = decltype(nb_const)::value;
      constexpr int NDS0 = decltype(nds0_const)::value;
      constexpr int V = decltype(v_const)::value;
      constexpr int V0 = decltype(v0_const)::value;
      if (NDS0 > 0) __builtin_amdgcn_sched_group_barrier(0x100, NDS0, 0);
      if (NBLK > 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int m = 0; m < NB; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, V0, 0);
        }
      }
#pragma unroll
      for (int b = 1; b < NBLK; ++b) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int m = 0; m < NB; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
        }
      }
    };

    // tile start: chunk 0 landed (weights in the slot, activations in buffer cb) and chunk 1's
    // activations in flight; the weights of chunk 0 go to registers, those of chunk 1 into the slot
    const Ctx cur = make_ctx(fetch(par));
    uint32_t aoff[A_ITERS];
    row_offsets(aoff);
    uint4 bq[NB];
    uint32_t sc[NB];
    read_w(bq, sc);
    wait_lds_reads();
    if (nK > 1) issue_w(cur, 1);
#pragma unroll
    for (int f = 0; f < NB; ++f) wcur[f] = w_op(bq[f], sc[f], 0);
    // Invariant at the top of chunk c: bq/sc hold chunk c's weights, wcur the operands of its
    // first MFMA step and xs that step's first D activation fragments; loads in flight, oldest
    // first: the activations, then the weights, of chunk c + 1 (of this tile or, past its end, the
    // next tile's activations of its chunk 0, then its weights of chunk 0).
    OpT xs[D];
#pragma unroll
    for (int d = 0; d < D; ++d) xs[d] = frag(lds + cb * A_BYTES, 0, d);
    // zero, opaque and distinct per RB: otherwise code generation merges the identical clearing of
    // every variant into one place and holds a second set of accumulators beside the previous
    // tile's, which do not fit in the registers
    f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    asm volatile("; zero rb %1" : "+v"(zero) : "n"(RB));
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int f = 0; f < NB; ++f) acc[i][f] = zero;
    has_next = false;

    auto chunk = [&](int c, auto mode_const) {
      constexpr int MODE = decltype(mode_const)::value;
      // loads this chunk issues: this tile's chunk c + 2 (MID), the next tile's chunk c + 2 - nK
      // (PEN, LAST, when there is a next tile)
      const bool loads = MODE == MID || has_next;
      // step 3 reads the following chunk's weights and first activation fragments (this tile's)
      constexpr bool NEXT = MODE != LAST;
      int bc = cb + c % NA;
      if (bc >= NA) bc -= NA;
      const uint8_t* abuf = lds + bc * A_BYTES;
      const uint8_t* anext = lds + (bc == NA - 1 ? 0 : bc + 1) * A_BYTES;
      const int b2 = bc == 0 ? NA - 1 : bc - 1;   // (bc + 2) % 3: the buffer chunk c - 1 used
      if constexpr (MODE == MID) {
        if (chain) hook_top(c);
        issue_a(cur, aoff, c + 2, b2);
      }
      // the next tile's operand bases (PEN, LAST)
      const Ctx nxt = MODE == MID ? cur : make_ctx(fetch(par ^ 1));
      if (MODE != MID && loads) {
        uint32_t ao[A_ITERS];
        row_offsets(ao);
        issue_a(nxt, ao, c + 2 - nK, b2);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < STEPS; ++j) {
        OpT x[RB + D];
        OpT wnext[NB];
#pragma unroll
        for (int d = 0; d < D; ++d) x[d] = xs[d];
        if (j + 1 < STEPS) {
#pragma unroll
          for (int f = 0; f < NB; ++f) wnext[f] = w_op(bq[f], sc[f], j + 1);
          blocks(IntC<0>{}, IntC<RB>{}, x, abuf, j, abuf, j + 1, IntC<1>{});
          pin(wnext);
          interleave(IntC<RB>{}, IntC<0>{}, IntC<VPM>{}, IntC<VPM>{});
          __builtin_amdgcn_sched_barrier(0);
        } else if constexpr (NEXT) {
          // this wave's activations and weights of the following chunk have landed (only the
          // activations issued at the top of this chunk may be in flight); the weights go from the
          // wave's own slot to registers and are dequantized for the following chunk's first step
          if (loads) wait_vm(IntC<A_ITERS>{});
          else wait_vm(IntC<0>{});
          read_w(bq, sc);
#pragma unroll
          for (int f = 0; f < NB; ++f) wnext[f] = w_op(bq[f], sc[f], 0);
          blocks(IntC<0>{}, IntC<H1>{}, x, abuf, j, anext, 0, IntC<0>{});
          pin(wnext);
          interleave(IntC<H1>{}, IntC<2 * NB>{}, IntC<VPM_A>{}, IntC<0>{});
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (MODE == MID) {
            if (chain) hook_mid(c);
          }
          // the slot is free again: the weights two chunks ahead go into it; after the barrier
          // every wave's activations of the following chunk are in LDS and every read of this
          // chunk's buffer has returned
          wait_lds_reads();
          if constexpr (MODE == MID) issue_w(cur, c + 2);
          else if (loads) issue_w(nxt, c + 2 - nK);
          __syncthreads();
          blocks(IntC<H1>{}, IntC<RB>{}, x, abuf, j, anext, 0, IntC<1>{});
          interleave(IntC<RB - H1>{}, IntC<0>{}, IntC<VPM>{}, IntC<VPM>{});
          __builtin_amdgcn_sched_barrier(0);
        } else {
          blocks(IntC<0>{}, IntC<RB>{}, x, abuf, j, abuf, j, IntC<0>{});
          // the next tile's chunk 0 has landed (this wave's share; its activations of chunk 1 may
          // be in flight); after the barrier every wave's share is in LDS and every read of this
          // chunk's buffer has returned
          if (loads) wait_vm(IntC<A_ITERS>{});
          wait_lds_reads();
          __syncthreads();
        }
        if (j + 1 < STEPS || NEXT) {
#pragma unroll
          for (int f = 0; f < NB; ++f) wcur[f] = wnext[f];
#pragma unroll
          for (int d = 0; d < D; ++d) xs[d] = x[RB + d];
        }
      }
    };
    for (int c = 0; c + 2 < nK; ++c) chunk(c, IntC<MID>{});
    if (nK > 1) chunk(nK - 2, IntC<PEN>{});
    chunk(nK - 1, IntC<LAST>{});
    // only the RB blocks with real rows are stored: the other accumulators are never live
    const Tile t = fetch(par);
    const auto* a = args();
    GemmProblem pe{};
    pe.N = a->N;
    pe.out = a->out;
    pe.out_tiled = a->out_tiled;
    pe.a_gscale = a->a_gscale;
    pe.h16 = H16 ? 1 : 0;
    pe.hshift_out = a->hshift_out;
    // the expert's global scales by scalar loads (through the constant address space: they are not
    // written while the kernel runs), which leave the direct loads in flight alone
    float g0 = 1.f, g1 = 1.f;
    if constexpr (WFmt<FMT>::kGlobalScale) {
      const float* gs = t.extra ? a->extra.gs : a->bank.gs;
      const int per = t.extra ? a->extra.gs_per_expert : a->bank.gs_per_expert;
      const auto* gk = (const __attribute__((address_space(4))) float*)(gs + (size_t)t.group * per);
      g0 = gk[0];
      if (GATE_UP) g1 = gk[1];
    }
    const TileInfo ti{t.group, t.row0, t.rows, t.a_row0, t.extra};
    if constexpr (A16)
      epilogue_at<MI, NB, GATE_UP, BN, COLS_PER_WAVE>(pe, g0, g1, ti, t.ntile, acc, t.mtile,
                                                      (const int*)s_shift[par], IntC<RB>{}, lane_now(), wave);
    else
      epilogue_at<MI, NB, GATE_UP, BN, COLS_PER_WAVE>(pe, g0, g1, ti, t.ntile, acc, t.mtile, nullptr, IntC<RB>{},
                                                      lane_now(), wave);
  };
  for (;;) {
    switch ((__builtin_amdgcn_readfirstlane(s_tile[par][3]) + 15) / 16) {
      case 1: run(IntC<1>{}); break;
      case 2: run(IntC<2>{}); break;
      case 3: run(IntC<3>{}); break;
      case 4: run(IntC<4>{}); break;
      case 5: run(IntC<5>{}); break;
      case 6: run(IntC<6>{}); break;
      case 7: run(IntC<7>{}); break;
      default: run(IntC<8>{}); break;
    }
    if (!has_next) break;
    // the next tile: its chunk 0 landed (buffer cb + nK), chunk 1's activations in flight; s_aoff
    // holds its rows
    par ^= 1;
    cb = (cb + nK) % NA;
  }
}

// Compute units of the current device (looked up once per device; 0 if the query fails).
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int NB, bool GATE_UP, int WAVES, int FMT>
moe_status_t launch_tall(const GemmProblem& p, hipStream_t stream) {
  constexpr int BN = WAVES * (GATE_UP ? 16 * (NB / 2) : 16 * NB);
  if (p.N % BN != 0 || p.K % kTallBK != 0) return MOE_ERR_INVALID_ARGUMENT;
  const int NT = p.N / BN;
  const long long mt = (p.G > 0 ? (long long)std::min(p.G, p.M) + p.M / kTallRows : 0LL) +
                       (p.has_extra ? (p.M_extra + kTallRows - 1) / kTallRows : 0);
  long long grid = mt * NT;
  if (grid == 0) return MOE_OK;
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  if constexpr (WAVES == 8) {
    if (p.G > kTallMaxGroups) return MOE_ERR_INVALID_ARGUMENT;
    // six K chunks or more: one workgroup per compute unit walks its tiles (shorter K: one tile per
    // workgroup, the kernel never chains)
    if (p.K / kTallBK >= 6) {
      const int cus = device_cus();
      if (cus <= 0) return MOE_ERR_HIP;
      grid = std::min(grid, (long long)std::max(kXcds, cus / kXcds * kXcds));
    }
    if constexpr (FMT == kFmtNvfp4) {
      // fp16 operand rows: the gate/up token rows, or h (down) when the gate/up launch wrote it as fp16
      if (GATE_UP && p.a16 && p.h16 && p.hshift_out && p.out_tiled) {
        hipLaunchKernelGGL((grouped_gemm_tall_lds_kernel<NB, GATE_UP, FMT, true, GATE_UP>), dim3((unsigned)grid),
                           dim3(512), 0, stream, p);
        return launch_status();
      }
      if (GATE_UP ? p.a16 != nullptr : (p.h16 && p.a16 && p.row_shift && p.a_tiled)) {
        hipLaunchKernelGGL((grouped_gemm_tall_lds_kernel<NB, GATE_UP, FMT, true>), dim3((unsigned)grid), dim3(512), 0,
                           stream, p);
        return launch_status();
      }
    }
    hipLaunchKernelGGL((grouped_gemm_tall_lds_kernel<NB, GATE_UP, FMT, false>), dim3((unsigned)grid), dim3(512), 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((grouped_gemm_tall_kernel<NB, GATE_UP, WAVES, FMT>), dim3((unsigned)grid), dim3(64 * WAVES), 0,
                       stream, p);
  }
  return launch_status();
}

template <int MI, int NB, int BK, bool GATE_UP, int FMT>
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
  hipLaunchKernelGGL((grouped_gemm_kernel<MI, NB, BK, GATE_UP, FMT>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return launch_status();
}

template <int NB, int BK, bool GATE_UP>
moe_status_t launch_skinny(const GemmProblem& p, hipStream_t stream) {
  constexpr int BN = GATE_UP ? 4 * 16 * (NB / 2) : 4 * 16 * NB;
  if (p.N % BN != 0 || p.K % BK != 0) return MOE_ERR_INVALID_ARGUMENT;
  const int NT = p.N / BN;
  const long long mt = (p.G > 0 ? (long long)std::min(p.G, p.M) + p.M / kSkinnyRows : 0LL) +
                       (p.has_extra ? (p.M_extra + kSkinnyRows - 1) / kSkinnyRows : 0);
  const long long grid = mt * NT;
  if (grid == 0) return MOE_OK;
  if (grid > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL((grouped_gemm_skinny_kernel<NB, BK, GATE_UP>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     p);
  return launch_status();
}

// 16-row tiles (up to 16 rows per expert on average; NVFP4 groups of at most 8 take the skinny
// kernel): 512-wide K chunks for long reductions, 256-wide for shorter ones (more workgroups in
// flight; measured on the decode-shaped down GEMM, K = 1536).
template <bool GATE_UP, int FMT>
moe_status_t launch_small(const GemmProblem& p, hipStream_t stream) {
  if (p.K % 512 == 0 && p.K >= 4096) return launch_cfg<1, 2, 512, GATE_UP, FMT>(p, stream);
  if (p.K % 256 == 0) return launch_cfg<1, 2, 256, GATE_UP, FMT>(p, stream);
  return launch_cfg<1, 2, 128, GATE_UP, FMT>(p, stream);
}

}  // namespace

namespace {
// rows per group on average decides the tile height
long long avg_rows(const GemmProblem& p) {
  const long long rows = (long long)p.M + (p.has_extra ? p.M_extra : 0);
  const long long groups = (long long)p.G + (p.has_extra ? 1 : 0);
  return groups ? rows / groups : 0;
}
}  // namespace

namespace {
template <int FMT>
moe_status_t launch_format(const GemmProblem& p, hipStream_t stream) {
  const bool gate_up = p.stage == MOE_GEMM_GATE_UP;
  const long long avg = avg_rows(p);
  // the skinny kernel applies E4M3 scales to per-group sums; MXFP4 needs no such trick (its scale
  // is applied by the conversion), so its few-row groups take the 16-row kernel
  if (FMT == kFmtNvfp4 && avg <= kSkinnyRows) {
    if (p.K % 256 == 0) return gate_up ? launch_skinny<2, 256, true>(p, stream) : launch_skinny<2, 256, false>(p, stream);
    return gate_up ? launch_skinny<2, 128, true>(p, stream) : launch_skinny<2, 128, false>(p, stream);
  }
  if (gate_up) {
    if (avg <= 16) return launch_small<true, FMT>(p, stream);
    if (avg <= 32) return launch_cfg<4, 4, 128, true, FMT>(p, stream);
    // eight waves (one workgroup per CU) where the width allows: half the A traffic per MFMA
    return (p.N % 256 == 0) ? launch_tall<4, true, 8, FMT>(p, stream) : launch_tall<4, true, 4, FMT>(p, stream);
  }
  const bool wide = (p.N % 256) == 0;
  if (avg <= 16) return launch_small<false, FMT>(p, stream);
  if (avg <= 32) return wide ? launch_cfg<4, 4, 128, false, FMT>(p, stream) : launch_cfg<4, 2, 128, false, FMT>(p, stream);
  // down: the eight-wave kernel's 512-column tiles where the width allows (one workgroup per CU
  // walking its tiles: 6% faster than the four-wave kernel with two workgroups per CU at both
  // prefill shapes, NVFP4; 5% for MXFP4), else four waves
  if (p.N % 512 == 0) return launch_tall<4, false, 8, FMT>(p, stream);
  return wide ? launch_tall<4, false, 4, FMT>(p, stream) : launch_tall<2, false, 4, FMT>(p, stream);
}
}  // namespace

bool grouped_gemm_uses_tall_tiles(const GemmProblem& p) { return avg_rows(p) > 32; }

// The skinny (8-row) tiles of launch_format: NVFP4 with at most 8 rows per group on average.
bool grouped_gemm_uses_skinny_tiles(const GemmProblem& p) {
  return p.bank.format == kFmtNvfp4 && avg_rows(p) <= kSkinnyRows;
}

// The eight-wave NVFP4 paths (launch_format) read fp16 rows: gate/up always, down when it is
// handed fp16 h (GemmProblem::h16).
bool grouped_gemm_takes_f16_rows(const GemmProblem& p) {
  if (p.bank.format != kFmtNvfp4 || !grouped_gemm_uses_tall_tiles(p)) return false;
  return p.stage == MOE_GEMM_GATE_UP ? p.N % 256 == 0 : p.N % 512 == 0;
}

namespace {
// One workgroup per row: the row's largest magnitude (NaN ignored), then the row times 2^xs in
// fp16 (round to nearest even), xs = 14 - floor(log2(max)) so that the largest magnitude lands
// in [2^14, 2^15): every bf16 element within 2^31 of it keeps all 8 significant bits (normal fp16
// down to 2^-14, subnormal steps of 2^-24).  A row of zeros or with an infinity keeps xs 0.  With
// the weight-row norm bounds ng, nu (fp16 h path), the same pass sums the squares of the scaled
// row and derives the power of two hs of the token's h rows (launch_act_to_f16); hs = 0 without
// them, for a row of zeros and for a non-finite row.
__global__ __launch_bounds__(256) void act_to_f16_kernel(const uint16_t* __restrict__ x, int H,
                                                         uint16_t* __restrict__ x16, int32_t* __restrict__ shift,
                                                         float ng, float nu) {
  __shared__ float wmax[4];
  __shared__ float wss[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* row = x + (size_t)blockIdx.x * H;
  float m = 0.f;
  for (int h = tid * 8; h < H; h += 256 * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + h);
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = fmaxf(m, fabsf(__uint_as_float(q[i] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(q[i] & 0xFFFF0000u)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int sh = (m > 0.f && m <= 3.4028235e38f) ? 14 - ilogbf(m) : 0;
  uint16_t* orow = x16 + (size_t)blockIdx.x * H;
  // sum of squares of the scaled row (each square exact, below 2^30; the sum rounds in fp32)
  float ss = 0.f;
  for (int h = tid * 8; h < H; h += 256 * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + h);
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = ldexpf(__uint_as_float(q[i] << 16), sh), b = ldexpf(__uint_as_float(q[i] & 0xFFFF0000u), sh);
      ss += a * a + b * b;
      const _Float16 lo = (_Float16)a;
      const _Float16 hi = (_Float16)b;
      o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<uint4*>(orow + h) = uint4{o[0], o[1], o[2], o[3]};
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) wss[wave] = ss;
  __syncthreads();
  if (tid == 0) {
    int hs = 0;
    if (ng > 0.f && nu > 0.f) {
      // ||x|| 2^sh, rounded up (1% covers the fp32 rounding of the sum and of the square root)
      const float n16 = sqrtf((wss[0] + wss[1]) + (wss[2] + wss[3])) * 1.01f;
      if (n16 > 0.f && n16 <= 3.4028235e38f && ng <= 3.4028235e38f && nu <= 3.4028235e38f) {
        // |g| 2^sh <= n16 ng and |u| 2^sh <= n16 nu, taken apart into mantissas in [0.5, 1) and
        // exponents so that nothing overflows; |silu(g)| = |g| sigmoid(g) <= |g| < 2^ea, |u| < 2^eb
        int a, b, c;
        const float fa = frexpf(n16, &a), fb = frexpf(ng, &b), fc = frexpf(nu, &c);
        const int ea = ilogbf(fa * fb) + 1 + a + b - sh;
        const int eb = ilogbf(fa * fc) + 1 + a + c - sh;
        // |h| < 2^(ea + eb); below 2^13 after the shift.  The clamp keeps every finite bf16 h
        // (below 2^128) within fp16 range
        hs = min(max(13 - ea - eb, -120), 120);
      }
    }
    shift[blockIdx.x] = (int32_t)(((uint32_t)sh & 0xFFFFu) | ((uint32_t)hs << 16));
  }
}
}  // namespace

moe_status_t launch_act_to_f16(const uint16_t* x, int32_t T, int32_t H, uint16_t* x16, int32_t* shift, float ng,
                               float nu, hipStream_t stream) {
  if (T < 0 || H <= 0 || H % 8 != 0) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  hipLaunchKernelGGL(act_to_f16_kernel, dim3((unsigned)T), dim3(256), 0, stream, x, (int)H, x16, shift, ng, nu);
  return launch_status();
}

moe_status_t launch_grouped_gemm(const GemmProblem& p, hipStream_t stream) {
  // the tiled activation layouts exist only on the 128-row path
  if ((p.a_tiled || p.out_tiled) && !grouped_gemm_uses_tall_tiles(p)) return MOE_ERR_INVALID_ARGUMENT;
  if (p.out_tiled && p.stage != MOE_GEMM_GATE_UP) return MOE_ERR_INVALID_ARGUMENT;
  if (p.has_extra && p.extra.format != p.bank.format) return MOE_ERR_INVALID_ARGUMENT;
  if (p.bank.format == kFmtMxfp4) return launch_format<kFmtMxfp4>(p, stream);
  if (p.bank.format == kFmtNvfp4) return launch_format<kFmtNvfp4>(p, stream);
  return MOE_ERR_INVALID_ARGUMENT;
}

}  // namespace moe
