// Combine (S6) of the NVFP4 MoE layer, gfx950: one workgroup per (token, 2048-column slice), each
// thread 8 consecutive columns (combine_row.h).
#include "combine_row.h"

namespace moe {
namespace {

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const uint16_t* __restrict__ y,
                                                                  const int32_t* __restrict__ slot_to_row,
                                                                  const float* __restrict__ w,
                                                                  const uint16_t* __restrict__ y_shared, int k,
                                                                  int H, uint16_t* __restrict__ out) {
  const int h0 = blockIdx.x * kCombineCols + threadIdx.x * 8;
  if (h0 >= H) return;
  combine_cols(y, slot_to_row, w, y_shared, blockIdx.y, h0, k, H, out, false);
}

}  // namespace

moe_status_t launch_combine(const uint16_t* y_rows, const int32_t* slot_to_row, const float* w,
                            const uint16_t* y_shared, int32_t T, int32_t k, int32_t H, uint16_t* out,
                            hipStream_t stream) {
  if (T == 0) return MOE_OK;
  hipLaunchKernelGGL(combine_kernel, dim3((H + kCombineCols - 1) / kCombineCols, T), dim3(kCombineThreads), 0, stream,
                     y_rows, slot_to_row, w, y_shared, (int)k, (int)H, out);
  return launch_status();
}

}  // namespace moe
