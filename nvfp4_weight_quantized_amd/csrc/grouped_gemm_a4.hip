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
//  * Weights are the first operand, read in the W4A4 tile layout (layout.hip): one contiguous 1 KB
//    load per 16-row x 128-K tile and wave, plus one scale byte per lane.
//  * Activations (codes [rows][K/2], scales [rows][K/32], quantized by quantize.hip) are the second
//    operand.  Per 128-K chunk the 128-row tile's codes (8 KB, eight 1 KB fragments, one per wave)
//    and scales (one dword per row: its four blocks of the chunk, 512 B, loaded by waves 0 and 1)
//    go global -> LDS by direct loads (gathered through the sorted slot list for gate/up) into a
//    ring of three chunk buffers (two chunks in flight); each wave reads every fragment back with
//    one ds_read_b128 and its scale dword with one ds_read_b32, shifted to the lane's block.
//  * 128-row tiles, 8 waves; the same tile list, XCD-aware tile order and per-row-count main-loop
//    instantiations as the W4A16 tall-tile kernel (grouped_gemm.hip).
#include "common.h"
#include "gemm_tiles.h"

namespace moe {
namespace {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kA4Rows = 128;   // token rows per tile
constexpr int kA4Waves = 8;
constexpr int kA4Bufs = 3;     // LDS chunk buffers: the current chunk and two in flight

// acc[first-operand row 4q + r][second-operand row n] += (W * 2^ws) . (X * 2^xs) over 128 K.
__device__ __forceinline__ f32x4 mfma_fp4(const uint4& w, uint32_t ws, const uint4& x, uint32_t xs, const f32x4& acc) {
  const i32x8 a = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
  const i32x8 b = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  // format codes 4, 4: both operands E2M1 (only the first four registers are read)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 4, 0, (int)ws, 0, (int)xs);
}

__device__ __forceinline__ uint4 load_weights16(const uint8_t* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
}

template <int NB, bool GATE_UP>
__global__ __launch_bounds__(64 * kA4Waves, 1) void grouped_gemm_a4_kernel(GemmProblemA4 p) {
  constexpr int WAVES = kA4Waves;
  constexpr int MI = kA4Rows / 16;
  constexpr int BM = kA4Rows;
  constexpr int COLS_PER_WAVE = GATE_UP ? 16 * (NB / 2) : 16 * NB;
  constexpr int BN = WAVES * COLS_PER_WAVE;
  constexpr int BUF = MI * 1024;                 // one chunk: 8 fragments of 1 KB
  constexpr int SBUF = BM * 4;                   // one chunk's activation scales: a dword per row
  constexpr int NBUF = kA4Bufs;
  static_assert(MI == WAVES && BM == 128, "one activation fragment per wave, scales by waves 0 and 1");
  __shared__ __attribute__((aligned(1024))) uint8_t As[NBUF * BUF];
  __shared__ __attribute__((aligned(512))) uint8_t Ss[NBUF * SBUF];
  __shared__ uint32_t s_arow[BM];
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
  TileInfo ti;
  ti.group = __builtin_amdgcn_readfirstlane(tile.group);
  ti.row0 = __builtin_amdgcn_readfirstlane(tile.row0);
  ti.rows = __builtin_amdgcn_readfirstlane(tile.rows);
  ti.a_row0 = __builtin_amdgcn_readfirstlane(tile.a_row0);
  ti.extra = __builtin_amdgcn_readfirstlane(tile.extra);
  const int ntile = __builtin_amdgcn_readfirstlane(tile_n);
  const int mtile = __builtin_amdgcn_readfirstlane(tile_m);
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
  // this wave's direct loads: fragment `wave` (row 16*wave + n, code bytes [16q, +16) of the chunk)
  // and, for waves 0 and 1, the scale dwords (blocks [4c, 4c + 4)) of rows 64*wave + lane
  const uint32_t a_off = s_arow[16 * wave + nl] * (uint32_t)(K / 2) + (uint32_t)(16 * q);
  const bool loads_scales = wave < 2;
  const uint32_t s_off = loads_scales ? s_arow[64 * wave + lane] * (uint32_t)(K / 32) : 0u;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)As;
  const uint32_t lds_s0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)Ss;

  const int ktiles = K / 128;
  const size_t rows_per_expert = GATE_UP ? 2 * (size_t)p.N : (size_t)p.N;
  const uint8_t* wexp = bank.w + (size_t)ti.group * rows_per_expert * (size_t)(K / 2) + 16 * lane;
  const uint8_t* sexp = bank.ws + (size_t)ti.group * rows_per_expert * (size_t)(K / 32) + lane;
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
      bn[f] = load_weights16(wexp + t * 1024);
      sn[f] = sexp[t * 64];
    }
  };
  auto issue_a = [&](int c, int buf) {
    direct_load16(acodes, a_off + 64u * (uint32_t)c, lds0 + (uint32_t)(buf * BUF + wave * 1024));
    if (loads_scales) direct_load4(ascale, s_off + 4u * (uint32_t)c, lds_s0 + (uint32_t)(buf * SBUF + wave * 256));
  };
  // Waits: every load of the chunk in flight has landed (vmcnt 0), or all but this wave's newest
  // direct loads (the chunk two ahead: one load, two for the waves that also load scales).  The
  // prefetch registers are operands, so the compiler's own wait for them lands here.
  auto fence_regs = [&]() {
#pragma unroll
    for (int f = 0; f < NB; ++f)
      asm volatile("" : "+v"(bn[f].x), "+v"(bn[f].y), "+v"(bn[f].z), "+v"(bn[f].w), "+v"(sn[f]) : : "memory");
  };
  auto wait_all = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
    fence_regs();
  };
  auto wait_keep_ahead = [&]() {
    if (loads_scales)
      asm volatile("s_waitcnt vmcnt(2)" : : : "memory");
    else
      asm volatile("s_waitcnt vmcnt(1)" : : : "memory");
    fence_regs();
  };

  auto run = [&](auto rb_const) {
    constexpr int RB = decltype(rb_const)::value;
    issue_a(0, 0);
    load_b(0);
    if (nK > 1) {
      issue_a(1, 1);
      wait_keep_ahead();
    } else {
      wait_all();
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
      if (c + 2 < nK) issue_a(c + 2, (c + 2) % NBUF);
      const uint8_t* abuf = As + (c % NBUF) * BUF + 16 * lane;
      const uint8_t* sbuf = Ss + (c % NBUF) * SBUF + 4 * nl;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const uint4 x = *reinterpret_cast<const uint4*>(abuf + i * 1024);
        const uint32_t xs = *reinterpret_cast<const uint32_t*>(sbuf + 64 * i) >> (8 * q);   // this lane's block
#pragma unroll
        for (int f = 0; f < NB; ++f) acc[i][f] = mfma_fp4(bq[f], sc[f], x, xs, acc[i][f]);
        // one fragment read per row block in flight (bounds the live registers)
        __builtin_amdgcn_sched_barrier(0);
      }
      if (c + 2 < nK)
        wait_keep_ahead();
      else
        wait_all();
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
  if (p.bank.format != MOE_WEIGHT_MXFP4 || (p.has_extra && p.extra.format != MOE_WEIGHT_MXFP4))
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
