// Load-time repack of NVFP4 weights into the MFMA tile layout the grouped GEMMs read.
//
// The pages' fused-MoE kernels also swizzle checkpoint weights once into their MMA tile layout
// ("Serving Solar Open 2 on DGX Spark", "Supporting real NVFP4 checkpoints"); this is the CDNA4
// equivalent.  A tensor [rows][cols] (rows % 16 == 0, cols % 128 == 0) becomes a sequence of tiles
// t = (rows/16 block nb) * (cols/128) + (128-column chunk c).  In tile t, lane l = 16*q + n of a
// 16x16x32 bf16 MFMA operand owns row r = 16*nb + n:
//   nibbles: 1024 bytes; bytes [16*l + 4*j, 16*l + 4*j + 4) (j = 0..3, the MFMA k-step) are the
//            canonical bytes [64*c + 16*j + 4*q, +4) of row r, i.e. K [128c + 32j + 8q, +8);
//   scales:  128 bytes; bytes [8*n, 8*n + 8) are row r's eight scale bytes of the chunk in the
//            order g0 g2 g4 g6 g1 g3 g5 g7 (g = canonical scale byte 8*c + g), so the dword at
//            8*n + 4*(q >> 1) holds, in byte j, the scale of K [128c + 32j + 8q, +8).
// A wave therefore reads a whole tile with one contiguous 1 KB load (and 128 B of scales).
// The repack is a pure byte permutation (same total size as the canonical layout).  MXFP4 weights
// (E8M0 scales per 32 elements, "vLLM on the NVIDIA DGX Spark", section 6.4) use the same nibble
// tiles with 64 scale bytes per tile (pack_tiles_mx_kernel).
#include "common.h"

namespace moe {
namespace {

// One thread per (tile, lane): 16 nibble bytes; the first 16 lanes of a tile also move 8 scale bytes.
__global__ __launch_bounds__(256) void pack_tiles_kernel(const uint8_t* __restrict__ packed,
                                                         const uint8_t* __restrict__ scales, long long total_lanes,
                                                         int rows, int cols, uint8_t* __restrict__ tiled,
                                                         uint8_t* __restrict__ tiled_scales) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total_lanes) return;
  const long long tile = gid >> 6;
  const int l = (int)(gid & 63);
  const int ct = cols / 128;
  const long long tiles_per_tensor = (long long)(rows / 16) * ct;
  const long long b = tile / tiles_per_tensor;
  const long long t = tile - b * tiles_per_tensor;
  const int nb = (int)(t / ct);
  const int c = (int)(t - (long long)nb * ct);
  const int q = l >> 4, n = l & 15;
  const long long row = b * rows + 16LL * nb + n;
  const uint8_t* src = packed + row * (cols / 2) + 64 * c + 4 * q;
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const uint32_t*>(src + 16 * j);
  *reinterpret_cast<uint4*>(tiled + tile * 1024 + 16 * l) = uint4{w[0], w[1], w[2], w[3]};
  if (q == 0) {
    const uint2 sv = *reinterpret_cast<const uint2*>(scales + row * (cols / 16) + 8 * c);
    const uint32_t lo = sv.x, hi = sv.y;   // bytes g0..g3, g4..g7
    const uint32_t even = (lo & 0xFFu) | ((lo >> 8) & 0xFF00u) | ((hi << 16) & 0xFF0000u) | ((hi << 8) & 0xFF000000u);
    const uint32_t odd = ((lo >> 8) & 0xFFu) | ((lo >> 16) & 0xFF00u) | ((hi << 8) & 0xFF0000u) | (hi & 0xFF000000u);
    *reinterpret_cast<uint2*>(tiled_scales + tile * 128 + 8 * n) = uint2{even, odd};
  }
}

// MXFP4: the same nibble permutation; scales are one E8M0 byte per 32 elements, so a tile holds
// 64 scale bytes: bytes [4*n, 4*n + 4) are row r's canonical scale bytes [4*c, 4*c + 4), and byte j
// of that dword is the scale of MFMA step j (K [128c + 32j, +32)) for every lane of row r.
__global__ __launch_bounds__(256) void pack_tiles_mx_kernel(const uint8_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ scales, long long total_lanes,
                                                            int rows, int cols, uint8_t* __restrict__ tiled,
                                                            uint8_t* __restrict__ tiled_scales) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total_lanes) return;
  const long long tile = gid >> 6;
  const int l = (int)(gid & 63);
  const int ct = cols / 128;
  const long long tiles_per_tensor = (long long)(rows / 16) * ct;
  const long long b = tile / tiles_per_tensor;
  const long long t = tile - b * tiles_per_tensor;
  const int nb = (int)(t / ct);
  const int c = (int)(t - (long long)nb * ct);
  const int q = l >> 4, n = l & 15;
  const long long row = b * rows + 16LL * nb + n;
  const uint8_t* src = packed + row * (cols / 2) + 64 * c + 4 * q;
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const uint32_t*>(src + 16 * j);
  *reinterpret_cast<uint4*>(tiled + tile * 1024 + 16 * l) = uint4{w[0], w[1], w[2], w[3]};
  if (q == 0)
    *reinterpret_cast<uint32_t*>(tiled_scales + tile * 64 + 4 * n) =
        *reinterpret_cast<const uint32_t*>(scales + row * (cols / 32) + 4 * c);
}

// W4A4 tiles for the scaled FP4 MFMA (grouped_gemm_a4.hip): lane l = 16*q + n owns row r and the
// 32 elements K [128c + 32q, +32), one E8M0 block.  Nibble bytes [16*l, 16*l + 16) of tile t are
// row r's canonical bytes [64*c + 16*q, +16); scale byte l is row r's canonical scale byte 4*c + q.
__global__ __launch_bounds__(256) void pack_tiles_a4_kernel(const uint8_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ scales, long long total_lanes,
                                                            int rows, int cols, uint8_t* __restrict__ tiled,
                                                            uint8_t* __restrict__ tiled_scales) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total_lanes) return;
  const long long tile = gid >> 6;
  const int l = (int)(gid & 63);
  const int ct = cols / 128;
  const long long tiles_per_tensor = (long long)(rows / 16) * ct;
  const long long b = tile / tiles_per_tensor;
  const long long t = tile - b * tiles_per_tensor;
  const int nb = (int)(t / ct);
  const int c = (int)(t - (long long)nb * ct);
  const int q = l >> 4, n = l & 15;
  const long long row = b * rows + 16LL * nb + n;
  *reinterpret_cast<uint4*>(tiled + tile * 1024 + 16 * l) =
      *reinterpret_cast<const uint4*>(packed + row * (cols / 2) + 64 * c + 16 * q);
  tiled_scales[tile * 64 + l] = scales[row * (cols / 32) + 4 * c + q];
}

}  // namespace

moe_status_t launch_pack_tiles_a4(const uint8_t* packed, const uint8_t* scales, int32_t num_tensors, int32_t rows,
                                  int32_t cols, uint8_t* tiled, uint8_t* tiled_scales, hipStream_t stream) {
  const long long lanes = (long long)num_tensors * (rows / 16) * (cols / 128) * 64;
  if (lanes == 0) return MOE_OK;
  const long long blocks = (lanes + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(pack_tiles_a4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, packed, scales, lanes,
                     (int)rows, (int)cols, tiled, tiled_scales);
  return launch_status();
}

moe_status_t launch_pack_tiles_mx(const uint8_t* packed, const uint8_t* scales, int32_t num_tensors, int32_t rows,
                                  int32_t cols, uint8_t* tiled, uint8_t* tiled_scales, hipStream_t stream) {
  const long long lanes = (long long)num_tensors * (rows / 16) * (cols / 128) * 64;
  if (lanes == 0) return MOE_OK;
  const long long blocks = (lanes + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(pack_tiles_mx_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, packed, scales, lanes,
                     (int)rows, (int)cols, tiled, tiled_scales);
  return launch_status();
}

moe_status_t launch_pack_tiles(const uint8_t* packed, const uint8_t* scales, int32_t num_tensors, int32_t rows,
                               int32_t cols, uint8_t* tiled, uint8_t* tiled_scales, hipStream_t stream) {
  const long long lanes = (long long)num_tensors * (rows / 16) * (cols / 128) * 64;
  if (lanes == 0) return MOE_OK;
  const long long blocks = (lanes + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(pack_tiles_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, packed, scales, lanes, (int)rows,
                     (int)cols, tiled, tiled_scales);
  return launch_status();
}

}  // namespace moe
