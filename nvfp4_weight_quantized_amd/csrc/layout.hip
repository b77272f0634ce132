// Load-time repack of NVFP4 weights into the MFMA tile layout the grouped GEMMs read.
//
// The pages' fused-MoE kernels also swizzle checkpoint weights once into their MMA tile layout
// ("Serving Solar Open 2 on DGX Spark", "Supporting real NVFP4 checkpoints"); this is the CDNA4
// equivalent.  A tensor [rows][cols] (rows % 16 == 0, cols % 128 == 0) becomes a sequence of tiles
// t = (rows/16 block nb) * (cols/128) + (128-column chunk c); tile t holds
//   nibbles: 1024 bytes, lane l = 16*q + n at bytes [16*l, 16*l + 16) = row 16*nb + n,
//            canonical bytes [64*c + 16*q, 64*c + 16*q + 16) (K range [128c + 32q, 128c + 32q + 32))
//   scales:  128 bytes, lane l at bytes [2*l, 2*l + 2) = row 16*nb + n, scale bytes 8*c + 2*q, +1.
// A wave reading one tile therefore issues one contiguous 1 KB load and one contiguous 128 B load.
// The repack is a pure byte permutation (same total size as the canonical layout).
#include "common.h"

namespace moe {
namespace {

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
  const uint4 v = *reinterpret_cast<const uint4*>(packed + row * (cols / 2) + 64 * c + 16 * q);
  *reinterpret_cast<uint4*>(tiled + tile * 1024 + 16 * l) = v;
  const uint16_t s = *reinterpret_cast<const uint16_t*>(scales + row * (cols / 16) + 8 * c + 2 * q);
  *reinterpret_cast<uint16_t*>(tiled_scales + tile * 128 + 2 * l) = s;
}

}  // namespace

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
