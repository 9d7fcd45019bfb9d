// quant.hip -- per-token activation quantisation (a launch of its own for a
// large batch; a small batch quantises inside the fused prologue), per-row
// requantisation of the SwiGLU output into GEMM2's tiled operand.
//
// "MiniMax-M3 W8A8 inference on K100AI" (mhpq.cn/news/1068415) §3.2 and §6.4:
// activations are quantised per token (one outlier token must not set the
// range of the others) after the SmoothQuant rescaling; §4.3: consecutive
// matmuls stay in INT8, so the SwiGLU output is requantised per row before
// the down projection. The rule is in layer_device.h.
#include "layer_device.h"

namespace moe {
namespace {

// x bf16 [T][H] -> qx int8 [T][H], sx fp32 [T]. One wavefront per token;
// the row stays in registers (MAXC chunks of 8 values per lane) between its
// maximum and its codes. Rows of 4097..8192 channels keep the raw words and
// scale them twice, so there (kStage) the block first copies inv_s (32 KB
// at most) into LDS for its four tokens, instead of every token reading it
// twice through the caches.
constexpr int kInvStage = 8192;
template <bool kF8, int MAXC, bool kStage>
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t *__restrict__ x,
                                                        const float *__restrict__ inv_s,
                                                        int64_t T, int H,
                                                        int8_t *__restrict__ qx,
                                                        float *__restrict__ sx, ActClip ac) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if constexpr (kStage) {
    __shared__ __attribute__((aligned(16))) float sinv[kInvStage];
    for (int i = threadIdx.x; i < (H >> 2); i += 256)
      reinterpret_cast<v4f *>(sinv)[i] = reinterpret_cast<const v4f *>(inv_s)[i];
    __syncthreads();
    if (t < T) quant_token_row<MAXC>(x + t * H, sinv, H, qx + t * H, sx + t, ac, kF8);
  } else {
    if (t < T) quant_token_row<MAXC>(x + t * H, inv_s, H, qx + t * H, sx + t, ac, kF8);
  }
}

// h fp32 [rows][F] with row max |h| in amax (float bits) -> qh int8 stored
// fragment-tiled (16 rows x 64 k per 1 KB, the layout of the weights: the
// activation operand of GEMM2) and sh fp32 [rows]. Block = one 16-row tile x
// 512 columns (two halves of 256); thread = 16 consecutive values of one row,
// which quantise to exactly one 16-byte chunk of a tile. Rows past the padded row count are
// left alone; padding rows (max 0, h never written) get codes 0.
template <bool kF8>
__global__ __launch_bounds__(512) void requant_kernel(const float *__restrict__ h,
                                                      const uint32_t *__restrict__ amax_bits,
                                                      const int32_t *__restrict__ poffsets, int E,
                                                      int F, int8_t *__restrict__ qh,
                                                      float *__restrict__ sh) {
  const int rt = blockIdx.x;
  const int row = rt * 16 + ((threadIdx.x >> 4) & 15);
  if (row >= poffsets[E]) return;
  const int c0 = blockIdx.y * 512 + (threadIdx.x >> 8) * 256 + (threadIdx.x & 15) * 16;
  if (c0 >= F) return;
  const float amax = __uint_as_float(amax_bits[row]);
  const float qmax = kF8 ? kFp8Max : 127.0f;
  if (c0 == 0) sh[row] = amax / qmax;
  v4i q = {0, 0, 0, 0};
  // A zero maximum (a padding row, or h all zero) gives codes 0 without
  // reading h.
  if (amax > 0.0f) {
    const float rr = qmax / amax;
    const float *hr = h + (size_t)row * F + c0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const v4f v = *reinterpret_cast<const v4f *>(hr + 4 * w);
      const float vv[4] = {v[0], v[1], v[2], v[3]};
      q[w] = (int)codes4(vv, rr, kF8);
    }
  }
  const int kt = c0 >> 6, g = (c0 & 63) >> 4;
  *reinterpret_cast<v4i *>(qh + frag_tile(rt, kt, F) + ((g * 16 + (row & 15)) << 4)) = q;
}

}  // namespace

hipError_t launch_act_quant(const uint16_t *x, const float *inv_s, int64_t T, int H, int8_t *qx,
                            float *sx, ActClip ac, bool fp8, hipStream_t st, Timing tm) {
  const dim3 grid((unsigned)((T + 3) / 4));
  // rows up to 4096 channels fit eight 16-byte chunks per lane: half the
  // registers, twice the wavefronts in flight
  if (H <= 4096) {
    if (fp8) return launch_kernel(act_quant_kernel<true, 8, false>, grid, dim3(256), st, tm, x,
                                  inv_s, T, H, qx, sx, ac);
    return launch_kernel(act_quant_kernel<false, 8, false>, grid, dim3(256), st, tm, x, inv_s, T,
                         H, qx, sx, ac);
  }
  if (H <= kInvStage) {
    if (fp8) return launch_kernel(act_quant_kernel<true, 16, true>, grid, dim3(256), st, tm, x,
                                  inv_s, T, H, qx, sx, ac);
    return launch_kernel(act_quant_kernel<false, 16, true>, grid, dim3(256), st, tm, x, inv_s, T,
                         H, qx, sx, ac);
  }
  if (fp8) return launch_kernel(act_quant_kernel<true, 16, false>, grid, dim3(256), st, tm, x,
                                inv_s, T, H, qx, sx, ac);
  return launch_kernel(act_quant_kernel<false, 16, false>, grid, dim3(256), st, tm, x, inv_s, T, H,
                       qx, sx, ac);
}

hipError_t launch_requant(const float *h, const uint32_t *amax, const int32_t *poffsets, int E,
                          int64_t P, int F, int8_t *qh, float *sh, bool fp8, hipStream_t st,
                          Timing tm) {
  const dim3 grid((unsigned)((P + 15) / 16), (unsigned)((F + 511) / 512));
  if (fp8)
    return launch_kernel(requant_kernel<true>, grid, dim3(512), st, tm, h, amax, poffsets, E, F, qh,
                         sh);
  return launch_kernel(requant_kernel<false>, grid, dim3(512), st, tm, h, amax, poffsets, E, F, qh,
                       sh);
}

}  // namespace moe
