// combine.hip -- gate-weighted un-permute and sum of the expert outputs.
//
// "超大规模模型推理的Day0适配实践" §四: after the grouped GEMMs the MoE operator
// un-sorts the rows and takes the weighted sum per token (combine_2x4 and
// combine_2x8 in layer_device.h: fp32 in slot order, bfloat16 with ties to
// even). Grid (T, H/4096): one block covers 4096 outputs of one token.
//  - fp32 y rows (streaming path): 512 threads; thread i owns outputs
//    h + 4j.. and h + 1024 + 4j.., h = 2048 * (i / 256), j = i % 256, so each
//    wavefront load reads 1 KB of one y row.
//  - int16 y rows with a scale per 16 outputs (tiled path): 256 threads;
//    thread i owns outputs 8i.. and 2048 + 8i.. of the block's 4096, so each
//    wavefront code load reads 1 KB of one y row (plus the 4-byte scales,
//    one per two lanes), and stores 16 bytes per lane and group.
#include "layer_device.h"

namespace moe {
namespace {

__global__ __launch_bounds__(512) void combine_f32_kernel(const float *__restrict__ y,
                                                          const float *__restrict__ wts,
                                                          const int32_t *__restrict__ row_of,
                                                          int64_t T, int H, int k,
                                                          uint16_t *__restrict__ out) {
  const int n = blockIdx.y * 4096 + (threadIdx.x >> 8) * 2048 + (threadIdx.x & 255) * 4;
  if (n < H) combine_2x4(y, wts, row_of, blockIdx.x, H, k, n, n + 1024, out);
}

__global__ __launch_bounds__(256) void combine_y16_kernel(const YRows y,
                                                          const float *__restrict__ wts,
                                                          const int32_t *__restrict__ row_of,
                                                          int64_t T, int H, int k,
                                                          uint16_t *__restrict__ out) {
  const int n = blockIdx.y * 4096 + threadIdx.x * 8;
  if (n < H) combine_2x8(y, wts, row_of, blockIdx.x, H, k, n, n + 2048, out);
}

}  // namespace

hipError_t launch_combine(YRows y, const float *wts, const int32_t *row_of, int64_t T, int H,
                          int k, uint16_t *out, hipStream_t st, Timing tm) {
  const dim3 grid((unsigned)T, (unsigned)((H + 4095) / 4096));
  if (y.f)
    return launch_kernel(combine_f32_kernel, grid, dim3(512), st, tm, (const float *)y.f, wts,
                         row_of, T, H, k, out);
  return launch_kernel(combine_y16_kernel, grid, dim3(256), st, tm, y, wts, row_of, T, H, k, out);
}

}  // namespace moe
