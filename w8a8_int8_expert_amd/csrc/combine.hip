// combine.hip -- gate-weighted un-permute and sum of the expert outputs.
//
// "超大规模模型推理的Day0适配实践" §四: after the grouped GEMMs the MoE operator
// un-sorts the rows and takes the weighted sum per token. Here
//   out[t][n] = bf16( sum_{j < k, row_of[t*k+j] >= 0} w[t][j] * y[row][n] )
// accumulated in fp32 in slot order (so the result does not depend on
// scheduling), rounded to bfloat16 with ties to even. Dropped slots add
// nothing and the remaining weights are not renormalised.
// One block of 256 threads per token; each thread owns 4 consecutive
// outputs per 1024-wide stripe (16-byte loads of y, 8-byte stores of out).
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y,
                                                      const float *__restrict__ wts,
                                                      const int32_t *__restrict__ row_of,
                                                      int64_t T, int H, int k,
                                                      uint16_t *__restrict__ out) {
  __shared__ int32_t rows[kMaxTopK];
  __shared__ float ws[kMaxTopK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = row_of[t * k + threadIdx.x];
    ws[threadIdx.x] = wts[t * k + threadIdx.x];
  }
  __syncthreads();
  for (int n = threadIdx.x * 4; n < H; n += 1024) {
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) {
      const int32_t r = rows[j];
      if (r < 0) continue;
      const v4f v = *reinterpret_cast<const v4f *>(y + (int64_t)r * H + n);
      const float w = ws[j];
      acc[0] += w * v[0];
      acc[1] += w * v[1];
      acc[2] += w * v[2];
      acc[3] += w * v[3];
    }
    const uint32_t lo = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    *reinterpret_cast<uint2 *>(out + t * H + n) = make_uint2(lo, hi);
  }
}

}  // namespace

hipError_t launch_combine(const float *y, const float *wts, const int32_t *row_of, int64_t T,
                          int H, int k, uint16_t *out, hipStream_t st) {
  combine_kernel<<<dim3((unsigned)T), dim3(256), 0, st>>>(y, wts, row_of, T, H, k, out);
  return hipGetLastError();
}

}  // namespace moe
