// combine.hip -- gate-weighted un-permute and sum of the expert outputs.
//
// "超大规模模型推理的Day0适配实践" §四: after the grouped GEMMs the MoE operator
// un-sorts the rows and takes the weighted sum per token (combine_2x4 in
// layer_device.h: fp32 in slot order, bfloat16 with ties to even).
// Grid (T, H/4096), 512 threads per block covering 4096 outputs of one
// token (a whole y row of each slot at the prefill width): thread i owns
// outputs h + 4j.. and h + 1024 + 4j.., h = 2048 * (i / 256), j = i % 256,
// so each wavefront load reads 1 KB of one y row (two 16-byte loads per lane
// and kept slot, two 8-byte stores).
#include "layer_device.h"

namespace moe {
namespace {

__global__ __launch_bounds__(512) void combine_kernel(const float *__restrict__ y,
                                                      const float *__restrict__ wts,
                                                      const int32_t *__restrict__ row_of,
                                                      int64_t T, int H, int k,
                                                      uint16_t *__restrict__ out) {
  const int n = blockIdx.y * 4096 + (threadIdx.x >> 8) * 2048 + (threadIdx.x & 255) * 4;
  if (n < H) combine_2x4(y, wts, row_of, blockIdx.x, H, k, n, n + 1024, out);
}

}  // namespace

hipError_t launch_combine(const float *y, const float *wts, const int32_t *row_of, int64_t T,
                          int H, int k, uint16_t *out, hipStream_t st, Timing tm) {
  const dim3 grid((unsigned)T, (unsigned)((H + 4095) / 4096));
  return launch_kernel(combine_kernel, grid, dim3(512), st, tm, y, wts, row_of, T, H, k, out);
}

}  // namespace moe
