// quant.hip -- per-token activation quantisation and per-row requantisation
// as launches of their own (the multi-block path of a large batch; a small
// batch quantises inside the fused prologue, and the streaming GEMM1
// requantises in its last block per expert).
//
// "MiniMax-M3 W8A8 inference on K100AI" (mhpq.cn/news/1068415) §3.2 and §6.4:
// activations are quantised per token (one outlier token must not set the
// range of the others) after the SmoothQuant rescaling; §4.3: consecutive
// matmuls stay in INT8, so the SwiGLU output is requantised per row before
// the down projection. The rule is in layer_device.h.
#include "layer_device.h"

namespace moe {
namespace {

// x bf16 [T][H] -> qx int8 [T][H], sx fp32 [T]. One wavefront per token.
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t *__restrict__ x,
                                                        const float *__restrict__ inv_s,
                                                        int64_t T, int H,
                                                        int8_t *__restrict__ qx,
                                                        float *__restrict__ sx) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  quant_token_row<16>(x + t * H, inv_s, H, qx + t * H, sx + t);
}

// h fp32 [A][F] with row max |h| in amax (float bits) -> qh int8, sh fp32.
// Rows past the number of kept rows (offsets[E]) are left alone.
__global__ __launch_bounds__(256) void requant_kernel(const float *__restrict__ h,
                                                      const uint32_t *__restrict__ amax_bits,
                                                      const int32_t *__restrict__ offsets, int E,
                                                      int F, int8_t *__restrict__ qh,
                                                      float *__restrict__ sh) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= offsets[E]) return;
  requant_row(h + r * F, __uint_as_float(amax_bits[r]), F, qh + r * F, sh + r);
}

}  // namespace

hipError_t launch_act_quant(const uint16_t *x, const float *inv_s, int64_t T, int H, int8_t *qx,
                            float *sx, hipStream_t st, Timing tm) {
  return launch_kernel(act_quant_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), st, tm, x, inv_s,
                       T, H, qx, sx);
}

hipError_t launch_requant(const float *h, const uint32_t *amax, const int32_t *offsets, int E,
                          int64_t A, int F, int8_t *qh, float *sh, hipStream_t st, Timing tm) {
  return launch_kernel(requant_kernel, dim3((unsigned)((A + 3) / 4)), dim3(256), st, tm, h, amax,
                       offsets, E, F, qh, sh);
}

}  // namespace moe
