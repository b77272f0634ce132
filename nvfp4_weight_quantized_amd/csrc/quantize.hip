// On-device NVFP4 quantization of fp32 weights (weight preparation, not part of the layer pass),
// and of bf16 activation rows for the W4A4 variants.
//
// Recipe: group 16 along K, symmetric, FP8 E4M3 block scales, one fp32 global scale per tensor
// ("GLM-5.3-Flash-NVFP4 deployment blocked on SM121" discussion, compressed-tensors follow-up);
// block scales clamped to 448 ("Serving Solar Open 2 on DGX Spark", "Supporting real NVFP4
// checkpoints"); E2M1 elements of at most 6.0 packed two per byte ("vLLM on the NVIDIA DGX Spark",
// section 6.1).  Every step is an fp32 operation with round-to-nearest-even, done in this order:
//   t = amax_group / (6 * d);  t = min(t, 448);  s = E4M3_RNE(t)
//   q = w / (s * d) (0 when s * d == 0);  code = E2M1_RNE(q) saturated at 6, sign bit = (q < 0).
#include "common.h"

namespace moe {
namespace {

// Round t in [0, 448] to the nearest E4M3FN value (ties to even); returns the value and its byte.
__device__ __forceinline__ float e4m3_rne(float t, uint32_t* code) {
  if (!(t > 0.f)) {
    *code = 0;
    return 0.f;
  }
  int ex = ilogbf(t);                  // t in [2^ex, 2^(ex+1))
  const int qexp = max(ex, -6) - 3;    // grid spacing 2^qexp
  const float r = rintf(ldexpf(t, -qexp));
  const float v = ldexpf(r, qexp);     // exact
  if (v < 0x1p-6f) {                   // subnormal: m * 2^-9
    *code = (uint32_t)r;
  } else {
    const int ev = ilogbf(v);
    const uint32_t m = (uint32_t)(ldexpf(v, 3 - ev)) - 8u;   // v = (8 + m) * 2^(ev-3)
    *code = ((uint32_t)(ev + 7) << 3) | m;
  }
  return v;
}

// E2M1 code of q (nearest value, ties to even mantissa, saturating at 6); *mag receives the
// magnitude of the value it stands for.
__device__ __forceinline__ uint32_t e2m1_rne(float q, float* mag_out = nullptr) {
  const float mag = fabsf(q);
  const float step_inv = mag < 2.f ? 2.f : (mag < 4.f ? 1.f : 0.5f);
  const float v = fminf(rintf(mag * step_inv) / step_inv, 6.f);
  if (mag_out) *mag_out = v;
  uint32_t c;
  if (v <= 2.f) c = (uint32_t)(v * 2.f);        // 0, .5, 1, 1.5, 2 -> 0..4
  else if (v == 3.f) c = 5u;
  else if (v == 4.f) c = 6u;
  else c = 7u;
  return c | (q < 0.f ? 8u : 0u);
}

// One 16-element group with dequant global scale d: the packed codes (elements 0..7 in `lo`,
// low nibble first), the E4M3 byte of the block scale and (optionally) the values e2m1 * scale the
// codes stand for without the global scale -- at most 6 significant bits, so exact in fp32 and in
// any 16-bit float.
__device__ __forceinline__ void quantize_group16(const float (&v)[16], float d, uint32_t* lo, uint32_t* hi,
                                                 uint32_t* scode, float (*vals)[16] = nullptr) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  float t = __fdiv_rn(amax, __fmul_rn(6.0f, d));
  t = fminf(t, 448.0f);
  const float s = e4m3_rne(t, scode);
  const float sd = __fmul_rn(s, d);
  *lo = 0;
  *hi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float qv = (sd > 0.f) ? __fdiv_rn(v[i], sd) : 0.f;
    float mag;
    const uint32_t c = e2m1_rne(qv, &mag);
    if (i < 8) *lo |= c << (4 * i);
    else *hi |= c << (4 * (i - 8));
    if (vals) (*vals)[i] = (c & 8u) ? -(mag * s) : mag * s;
  }
}

// One thread per 16-element group.
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, long long groups_per_tensor,
                                                       long long total_groups, const float* __restrict__ gscale,
                                                       uint8_t* __restrict__ packed, uint8_t* __restrict__ scales) {
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= total_groups) return;
  const float d = gscale[g / groups_per_tensor];
  const float4* src = reinterpret_cast<const float4*>(w + g * 16);
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 x = src[i];
    v[4 * i] = x.x; v[4 * i + 1] = x.y; v[4 * i + 2] = x.z; v[4 * i + 3] = x.w;
  }
  uint32_t lo, hi, scode;
  quantize_group16(v, d, &lo, &hi, &scode);
  *reinterpret_cast<uint2*>(packed + g * 8) = uint2{lo, hi};
  scales[g] = (uint8_t)scode;
}

// NVFP4 activations (W4A4): bf16 rows quantized with the same rule and one dequant global scale d
// for the whole tensor (a static activation scale: "vLLM on the NVIDIA DGX Spark", section 6.1,
// one fp32 global scale for the activations; the fused MoE quantizes its bf16 inputs itself,
// section 4.3).  One thread per 16-element group; each output is optional: the packed codes, the
// E4M3 scale bytes, and the values e2m1 * block scale as bf16 (exact), which the W4A16 GEMMs take
// as their activation rows with the global scale applied in the epilogue.  `values` may be `a`
// itself: every thread reads its group before it writes it.
__global__ __launch_bounds__(256) void quantize_act_nv_kernel(const uint16_t* a, long long total_groups, float d,
                                                              uint8_t* __restrict__ packed,
                                                              uint8_t* __restrict__ scales, uint16_t* values) {
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= total_groups) return;
  const uint4* src = reinterpret_cast<const uint4*>(a + g * 16);
  float v[16];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint4 x = src[i];
    const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(u[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
    }
  }
  uint32_t lo, hi, scode;
  float vals[16];
  quantize_group16(v, d, &lo, &hi, &scode, &vals);
  if (packed) *reinterpret_cast<uint2*>(packed + g * 8) = uint2{lo, hi};
  if (scales) scales[g] = (uint8_t)scode;
  if (values) {
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      o[i] = (uint32_t)f32_to_bf16(vals[2 * i]) | ((uint32_t)f32_to_bf16(vals[2 * i + 1]) << 16);
    uint4* dst = reinterpret_cast<uint4*>(values + g * 16);
    dst[0] = uint4{o[0], o[1], o[2], o[3]};
    dst[1] = uint4{o[4], o[5], o[6], o[7]};
  }
}

// MXFP4 ("vLLM on the NVIDIA DGX Spark", section 6.4: E2M1 elements, one E8M0 exponent-only
// scale per 32 elements, no global scale).  One thread per 32-element group of fp32 weights or
// bf16 activations:
//   e = floor(log2(amax)) - 2 clamped to [-127, 127] (-127 when amax == 0), scale byte e + 127;
//   code = E2M1_RNE(|w| * 2^-e) saturated at 6 (exact power-of-two scaling), sign bit = (w < 0).
// The bf16 instantiation quantizes activation rows for the W4A4 GEMMs (W4A4 checkpoints carry
// 4-bit activations: "vLLM on the DGX Spark, the Hard Way", "The one rule that explains all the FP4
// confusion"; the fused MoE kernel quantizes bf16 hidden states itself: the guide's section 4.3).
__device__ __forceinline__ void load_group(const float* w, long long g, float (&v)[32]) {
  const float4* src = reinterpret_cast<const float4*>(w + g * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 x = src[i];
    v[4 * i] = x.x; v[4 * i + 1] = x.y; v[4 * i + 2] = x.z; v[4 * i + 3] = x.w;
  }
}

__device__ __forceinline__ void load_group(const uint16_t* a, long long g, float (&v)[32]) {
  const uint4* src = reinterpret_cast<const uint4*>(a + g * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 x = src[i];
    const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(u[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
    }
  }
}

template <typename In>
__global__ __launch_bounds__(256) void quantize_mx_kernel(const In* __restrict__ w, long long total_groups,
                                                          uint8_t* __restrict__ packed, uint8_t* __restrict__ scales) {
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= total_groups) return;
  float v[32];
  load_group(w, g, v);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = amax > 0.f ? min(max(ilogbf(amax) - 2, -127), 127) : -127;
  uint32_t word[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = e2m1_rne(ldexpf(fabsf(v[i]), -e)) | (v[i] < 0.f ? 8u : 0u);
    word[i >> 3] |= c << (4 * (i & 7));
  }
  *reinterpret_cast<uint4*>(packed + g * 16) = uint4{word[0], word[1], word[2], word[3]};
  scales[g] = (uint8_t)(e + 127);
}

// Norm bound of the fp16 h path (weight preparation): one wave per 16-row block of one expert's
// tiled w13 (gate rows, then up rows).  Lane l = 16q + n of the block's tile for K chunk c holds
// row n's elements [128c + 32j + 8q, +8) in its dword j, with the E4M3 scale in byte j of the
// tile's dword at 8n + 4(q >> 1) (the pack_tiles permutation).  Each row's squared Euclidean norm
// of E2M1 value times E4M3 scale is summed in fp64 (every term exact), its square root times the
// expert's gate or up global scale rounded up to fp32, and the largest over the block's rows folded
// into bound[0] (gate) or bound[1] (up) by an atomic maximum on the bits (non-negative floats order
// as their bit patterns; a NaN norm is ignored within the block, and a block of NaN norms leaves a
// NaN bound, which switches the fp16 h path off).
__global__ __launch_bounds__(256) void h16_bound_kernel(const uint8_t* __restrict__ w13,
                                                        const uint8_t* __restrict__ s13,
                                                        const float* __restrict__ gs, int E, int I, int H,
                                                        float* __restrict__ bound) {
  const int lane = threadIdx.x & 63;
  const long long nblk = (long long)E * (2 * I / 16);
  const long long blk = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= nblk) return;
  const int e = (int)(blk / (2 * I / 16)), nb = (int)(blk % (2 * I / 16));
  const int nc = H / 128;
  const uint8_t* wt = w13 + ((size_t)e * 2 * I + (size_t)nb * 16) * (size_t)(H / 2);
  const uint8_t* st = s13 + ((size_t)e * 2 * I + (size_t)nb * 16) * (size_t)(H / 16);
  const int q = lane >> 4, n = lane & 15;
  double ss = 0.0;
  for (int c = 0; c < nc; ++c) {
    const uint4 v = *reinterpret_cast<const uint4*>(wt + (size_t)c * 1024 + 16 * lane);
    const uint32_t sw = *reinterpret_cast<const uint32_t*>(st + (size_t)c * 128 + 8 * n + 4 * (q >> 1));
    const uint32_t words[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 squared, times 4: 0, 1, 4, 9, 16, 36, 64, 144
      int sq4 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = (words[j] >> (4 * i)) & 7;
        sq4 += m < 4 ? m * m : (m == 4 ? 16 : m == 5 ? 36 : m == 6 ? 64 : 144);
      }
      const float scf = j == 0   ? __builtin_amdgcn_cvt_f32_fp8((int)sw, 0)
                        : j == 1 ? __builtin_amdgcn_cvt_f32_fp8((int)sw, 1)
                        : j == 2 ? __builtin_amdgcn_cvt_f32_fp8((int)sw, 2)
                                 : __builtin_amdgcn_cvt_f32_fp8((int)sw, 3);
      const double sc = (double)scf;
      ss += 0.25 * (double)sq4 * sc * sc;
    }
  }
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  const int up = nb * 16 >= I ? 1 : 0;
  double r = sqrt(ss) * fabs((double)gs[2 * e + up]);
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) r = fmax(r, __shfl_xor(r, off));
  if (lane == 0) {
    float f = (float)r;
    if ((double)f < r) f = nextafterf(f, __builtin_inff());
    atomicMax(reinterpret_cast<unsigned int*>(bound) + up, __float_as_uint(f));
  }
}

}  // namespace

moe_status_t launch_h16_bound(const uint8_t* w13, const uint8_t* s13, const float* gs, int32_t E, int32_t I,
                              int32_t H, float* bound, hipStream_t stream) {
  if (E < 0 || I <= 0 || I % 16 != 0 || H <= 0 || H % 128 != 0) return MOE_ERR_INVALID_ARGUMENT;
  const long long waves = (long long)E * (2 * I / 16);
  if (waves == 0) return MOE_OK;
  const long long blocks = (waves + 3) / 4;
  if (blocks > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(h16_bound_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w13, s13, gs, (int)E, (int)I,
                     (int)H, bound);
  return launch_status();
}

moe_status_t launch_quantize_mx(const float* w, int32_t num_tensors, int32_t rows, int32_t cols, uint8_t* packed,
                                uint8_t* scales, hipStream_t stream) {
  const long long total = (long long)num_tensors * rows * (cols / 32);
  if (total == 0) return MOE_OK;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(quantize_mx_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, w, total, packed, scales);
  return launch_status();
}

moe_status_t launch_quantize_act_mx(const uint16_t* a, int64_t rows, int32_t cols, uint8_t* packed, uint8_t* scales,
                                    hipStream_t stream) {
  const long long total = (long long)rows * (cols / 32);
  if (total == 0) return MOE_OK;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(quantize_mx_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream, a, total, packed,
                     scales);
  return launch_status();
}

moe_status_t launch_quantize_act_nv(const uint16_t* a, int64_t rows, int32_t cols, float d, uint8_t* packed,
                                    uint8_t* scales, uint16_t* values, hipStream_t stream) {
  if (rows < 0 || cols < 0 || cols % 16 != 0) return MOE_ERR_INVALID_ARGUMENT;
  const long long total = (long long)rows * (cols / 16);
  if (total == 0) return MOE_OK;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(quantize_act_nv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, total, d, packed, scales,
                     values);
  return launch_status();
}

moe_status_t launch_quantize(const float* w, int32_t num_tensors, int32_t rows, int32_t cols,
                             const float* gscale, uint8_t* packed, uint8_t* scales, hipStream_t stream) {
  const long long gpt = (long long)rows * (cols / 16);
  const long long total = gpt * num_tensors;
  if (total == 0) return MOE_OK;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return MOE_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, gpt, total, gscale, packed,
                     scales);
  return launch_status();
}

}  // namespace moe
