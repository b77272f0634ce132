// W4A4 grouped GEMMs of the MoE layer (gate/up with SiLU(gate)*up, down) on the scaled FP4 matrix
// cores of gfx950: MXFP4 weights times MXFP4 activations, fp32 accumulation.
//
// Method: a W4A4 checkpoint carries 4-bit weights and 4-bit activations and runs a native FP4
// matmul, whose gain is in the compute-bound prefill regime ("vLLM on the DGX Spark, the Hard Way:
// Seven Months of GB10 Field Notes", sections "The one rule that explains all the FP4 confusion"
// and "Measured: native FP4 + MTP vs the published Marlin numbers"); both operands here are in the
// MXFP4 format ("vLLM on the NVIDIA DGX Spark: A Complete Technical Guide", section 6.4: E2M1
// elements, one E8M0 scale per 32 elements along K).
//
// CDNA4 design:
//  * One v_mfma_scale_f32_16x16x128_f8f6f4 per (16 weight rows, 16 token rows, 128 K), both
//    operands E2M1.  Operand layout (checked on the GPU against a CPU product): lane l = 16q + n
//    supplies row n's elements K [32q, +32) of the step as 16 bytes in canonical nibble order
//    (4 registers), and the E8M0 scale of that 32-block in the byte of its scale register that
//    op_sel picks (byte 0 here); lane l, register r of the result is row 4q + r of the first
//    operand and row n of the second -- the layout of the bf16 16x16 MFMAs, so the W4A16 epilogue
//    applies unchanged.  The scales are applied inside the instruction: no dequantization at all.
//  * Every operand goes global -> LDS by direct loads (global_load_lds_*), into a ring of three
//    chunk buffers with two 128-K chunks in flight; nothing is prefetched through registers, so
//    the bytes in flight per CU (about 84 KB) are set by LDS, not by the register budget -- the
//    weight stream needs them: at these shapes the kernel streams weights at HBM speed while its
//    matrix work takes a quarter of the time.  Per chunk and wave: the 1 KB activation fragment
//    of its 16 rows (codes [rows][K/2] from quantize.hip, gathered through the sorted slot list for
//    gate/up), its NB 1 KB weight tiles (W4A4 tile layout, layout.hip) and their 64 scale bytes
//    each (one 4-byte load per lane), and for waves 0 and 1 the activation scale dwords of 64 rows
//    (the row's four blocks of the chunk).  Each wave then reads its weight tiles once and every
//    activation fragment with one ds_read_b128 (scale: one ds_read_b32, shifted to the lane's
//    block).
//  * Tile order: within an expert the 128-row m-tiles of one output-column tile run next to each
//    other (blocks of up to 8 m-tiles, n-tiles inside a block), so the expert's weight tile is
//    fetched from HBM once and shared through L2 by the m-tiles running at the same time, while
//    the block's activation rows stay in L2 across the n-tiles.  Blocks and groups are spread over
//    the XCDs in contiguous ranges (workgroup b runs on XCD b mod 8).
//  * 128-row tiles, 8 waves; the same tile list, per-row-count main-loop instantiations and
//    epilogue as the W4A16 tall-tile kernel (grouped_gemm.hip).
#include "common.h"
#include "gemm_tiles.h"

namespace moe {
namespace {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kA4Rows = 128;   // token rows per tile
constexpr int kA4Waves = 8;
constexpr int kA4Bufs = 3;     // LDS chunk buffers: the current chunk and two in flight
constexpr int kA4Block = 8;    // m-tiles per block of the tile order

// acc[first-operand row 4q + r][second-operand row n] += (W * 2^ws) . (X * 2^xs) over 128 K.
__device__ __forceinline__ f32x4 mfma_fp4(const uint4& w, uint32_t ws, const uint4& x, uint32_t xs, const f32x4& acc) {
  const i32x8 a = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
  const i32x8 b = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  // format codes 4, 4: both operands E2M1 (only the first four registers are read)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 4, 0, (int)ws, 0, (int)xs);
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <int NB, bool GATE_UP>
__global__ __launch_bounds__(64 * kA4Waves, 1) void grouped_gemm_a4_kernel(GemmProblemA4 p) {
  constexpr int WAVES = kA4Waves;
  constexpr int MI = kA4Rows / 16;
  constexpr int BM = kA4Rows;
  constexpr int COLS_PER_WAVE = GATE_UP ? 16 * (NB / 2) : 16 * NB;
  constexpr int BN = WAVES * COLS_PER_WAVE;
  // one chunk buffer: activation codes (8 fragments of 1 KB), activation scales (a dword per
  // row), the waves' weight tiles (NB KB each) and weight scales (256 B each)
  constexpr int A_OFF = 0;
  constexpr int S_OFF = A_OFF + MI * 1024;
  constexpr int W_OFF = S_OFF + BM * 4;
  constexpr int WS_OFF = W_OFF + WAVES * NB * 1024;
  constexpr int BUF = WS_OFF + WAVES * 256;
  constexpr int NBUF = kA4Bufs;
  // direct loads per chunk: codes + NB weight tiles + weight scales (+ activation scales: waves 0, 1)
  constexpr int LOADS = NB + 2;
  static_assert(MI == WAVES && BM == 128 && NB <= 4, "one activation fragment per wave, scales by waves 0 and 1");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * BUF];
  __shared__ uint32_t s_arow[BM];
  __shared__ TileInfo tile;
  __shared__ int2 tile_span;
  __shared__ int tile_ok;
  __shared__ int tile_n;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4;
  const int nl = lane & 15;
  const int NT = p.N / BN;

  // tile lookup: L -> the group owning standard m-tile L / NT, then (m, n) inside the group in
  // the blocked order
  if (wave == 0) {
    const int total = count_tiles<BM>(p) * NT;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    const int L = (blockIdx.x % kXcds) * per_xcd + slot;
    bool ok = slot < per_xcd && L < total;
    if (ok) ok = find_tile<BM>(p, L / NT, &tile, &tile_span);
    if (lane == 0) {
      tile_ok = ok ? 1 : 0;
      tile_n = L;
    }
  }
  __syncthreads();
  if (!tile_ok) return;
  TileInfo ti;
  ti.group = __builtin_amdgcn_readfirstlane(tile.group);
  ti.extra = __builtin_amdgcn_readfirstlane(tile.extra);
  int ntile, mtile;
  {
    const int L = __builtin_amdgcn_readfirstlane(tile_n);
    const int within = __builtin_amdgcn_readfirstlane(tile_span.x);
    const int cnt = __builtin_amdgcn_readfirstlane(tile_span.y);
    const int mt_g = (cnt + BM - 1) / BM;
    const int base = L / NT - within;                   // the group's first standard m-tile
    const int local = L - base * NT;                    // in [0, mt_g * NT)
    const int blk = local / (kA4Block * NT);
    const int gm = min(kA4Block, mt_g - blk * kA4Block);
    const int r = local - blk * kA4Block * NT;
    const int m = blk * kA4Block + r % gm;
    ntile = r / gm;
    mtile = base + m;
    const int row0 = __builtin_amdgcn_readfirstlane(tile.row0) - within * BM;
    const int a_row0 = __builtin_amdgcn_readfirstlane(tile.a_row0) - within * BM;
    ti.row0 = row0 + m * BM;
    ti.a_row0 = a_row0 + m * BM;
    ti.rows = min(BM, cnt - m * BM);
  }
  const GemmBank& bank = ti.extra ? p.extra : p.bank;
  const int K = p.K;
  const int nK = K / 128;

  // source row of each tile row (rows past the group repeat its last row)
  const uint8_t* acodes = ti.extra ? p.a_extra : p.a;
  const uint8_t* ascale = ti.extra ? p.a_extra_scale : p.a_scale;
  if (tid < BM) {
    const int R = ti.a_row0 + min(tid, ti.rows - 1);
    s_arow[tid] = (uint32_t)((!ti.extra && p.row_index) ? p.row_index[R] / p.row_divisor : R);
  }
  __syncthreads();
  const bool loads_scales = wave < 2;
  // per-lane global byte offsets of this wave's direct loads (chunk 0)
  const uint32_t a_off = s_arow[16 * wave + nl] * (uint32_t)(K / 2) + (uint32_t)(16 * q);
  const uint32_t s_off = loads_scales ? s_arow[64 * wave + lane] * (uint32_t)(K / 32) : 0u;
  const int ktiles = K / 128;
  const size_t rows_per_expert = GATE_UP ? 2 * (size_t)p.N : (size_t)p.N;
  const uint8_t* wexp = bank.w + (size_t)ti.group * rows_per_expert * (size_t)(K / 2);
  const uint8_t* sexp = bank.ws + (size_t)ti.group * rows_per_expert * (size_t)(K / 32);
  uint32_t w_off[NB];
#pragma unroll
  for (int f = 0; f < NB; ++f)
    w_off[f] = (uint32_t)(frag_row_block<NB, GATE_UP, BN, COLS_PER_WAVE>(f, ntile, wave, p.N) * ktiles) * 1024u +
               (uint32_t)(16 * lane);
  // weight scales: lane l loads the 4 bytes [4(l%16), +4) of fragment (l/16) % NB's 64-byte tile
  const int sf = (lane >> 4) % NB;
  const uint32_t ws_off =
      (uint32_t)(frag_row_block<NB, GATE_UP, BN, COLS_PER_WAVE>(sf, ntile, wave, p.N) * ktiles) * 64u +
      (uint32_t)(4 * nl);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

  f32x4 acc[MI][NB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int f = 0; f < NB; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int c) {
    const uint32_t buf = lds0 + (uint32_t)((c % NBUF) * BUF);
    const uint32_t cc = (uint32_t)c;
    direct_load16(acodes, a_off + 64u * cc, buf + A_OFF + wave * 1024);
#pragma unroll
    for (int f = 0; f < NB; ++f) direct_load16(wexp, w_off[f] + 1024u * cc, buf + W_OFF + (wave * NB + f) * 1024);
    direct_load4(sexp, ws_off + 64u * cc, buf + WS_OFF + wave * 256);
    if (loads_scales) direct_load4(ascale, s_off + 4u * cc, buf + S_OFF + wave * 256);
  };
  // all but the newest chunk's loads have landed (the loads of one chunk are issued together)
  auto wait_keep_newest = [&]() {
    if (loads_scales)
      wait_vmcnt<LOADS + 1>();
    else
      wait_vmcnt<LOADS>();
  };

  auto run = [&](auto rb_const) {
    constexpr int RB = decltype(rb_const)::value;
    issue(0);
    if (nK > 1) {
      issue(1);
      wait_keep_newest();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    for (int c = 0; c < nK; ++c) {
      if (c + 2 < nK) issue(c + 2);
      const uint8_t* buf = lds + (c % NBUF) * BUF;
      uint4 wq[NB];
      uint32_t ws[NB];
#pragma unroll
      for (int f = 0; f < NB; ++f) {
        wq[f] = *reinterpret_cast<const uint4*>(buf + W_OFF + (wave * NB + f) * 1024 + 16 * lane);
        ws[f] = buf[WS_OFF + wave * 256 + f * 64 + lane];
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const uint4 x = *reinterpret_cast<const uint4*>(buf + A_OFF + i * 1024 + 16 * lane);
        const uint32_t xs = *reinterpret_cast<const uint32_t*>(buf + S_OFF + 4 * (16 * i + nl)) >> (8 * q);
#pragma unroll
        for (int f = 0; f < NB; ++f) acc[i][f] = mfma_fp4(wq[f], ws[f], x, xs, acc[i][f]);
      }
      if (c + 2 < nK)
        wait_keep_newest();
      else
        wait_vmcnt<0>();
      __syncthreads();
    }
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
  epilogue<MI, NB, GATE_UP, BN, COLS_PER_WAVE, false>(p, bank, ti, ntile, acc, mtile);
}

template <int NB, bool GATE_UP>
moe_status_t launch_a4(const GemmProblemA4& p, hipStream_t stream) {
  constexpr int BN = kA4Waves * (GATE_UP ? 16 * (NB / 2) : 16 * NB);
  if (p.N % BN != 0 || p.K % 128 != 0) return MOE_ERR_INVALID_ARGUMENT;
  const int NT = p.N / BN;
  const long long mt = (p.G > 0 ? (long long)std::min(p.G, p.M) + p.M / kA4Rows : 0LL) +
                       (p.has_extra ? (p.M_extra + kA4Rows - 1) / kA4Rows : 0);
  long long grid = mt * NT;
  if (grid == 0) return MOE_OK;
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL((grouped_gemm_a4_kernel<NB, GATE_UP>), dim3((unsigned)grid), dim3(64 * kA4Waves), 0, stream, p);
  return launch_status();
}

}  // namespace

moe_status_t launch_grouped_gemm_a4(const GemmProblemA4& p, hipStream_t stream) {
  if (p.bank.format != MOE_WEIGHT_MXFP4_A4 || (p.has_extra && p.extra.format != MOE_WEIGHT_MXFP4_A4))
    return MOE_ERR_INVALID_ARGUMENT;
  if (p.out_tiled) return MOE_ERR_INVALID_ARGUMENT;
  if (p.stage == MOE_GEMM_GATE_UP) {
    if (p.N % 256 == 0) return launch_a4<4, true>(p, stream);
    return launch_a4<2, true>(p, stream);
  }
  if (p.N % 512 == 0) return launch_a4<4, false>(p, stream);
  if (p.N % 256 == 0) return launch_a4<2, false>(p, stream);
  return launch_a4<1, false>(p, stream);
}

}  // namespace moe
