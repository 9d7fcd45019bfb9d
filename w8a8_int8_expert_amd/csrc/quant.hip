// quant.hip -- per-token activation quantisation and per-row requantisation.
//
// "MiniMax-M3 W8A8 inference on K100AI" (mhpq.cn/news/1068415) §3.2 and §6.4:
// activations are quantised per token (one outlier token must not set the
// range of the others) after the SmoothQuant rescaling; §4.3: consecutive
// matmuls stay in INT8, so the SwiGLU output is requantised per row before
// the down projection. Both use the symmetric absmax rule
//   amax = max |v|,  code = rint(fl32(v * fl32(127/amax))) in [-127, 127],
//   scale = amax/127  (an all-zero row: scale 0, codes 0),
// with every product rounded to fp32 so that codes are reproducible bit for
// bit. One wavefront per row; 16-byte coalesced loads and stores.
#include "moe_internal.h"

namespace moe {
namespace {

// x bf16 [T][H] -> qx int8 [T][H], sx fp32 [T]; xs = fl32(x * inv_s).
// Two passes over the row (the second hits L2): max, then codes.
__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t *__restrict__ x,
                                                        const float *__restrict__ inv_s,
                                                        int64_t T, int H,
                                                        int8_t *__restrict__ qx,
                                                        float *__restrict__ sx) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint16_t *xr = x + t * H;
  const int nchunk = H >> 3;  // 8 elements (16 bytes of bf16) per chunk
  float amax = 0.0f;
  for (int c = lane; c < nchunk; c += 64) {
    const v4i raw = *reinterpret_cast<const v4i *>(xr + c * 8);
    const v4f s0 = *reinterpret_cast<const v4f *>(inv_s + c * 8);
    const v4f s1 = *reinterpret_cast<const v4f *>(inv_s + c * 8 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = (uint32_t)raw[i];
      const float lo = __uint_as_float(w << 16) * (i < 2 ? s0[2 * i] : s1[2 * i - 4]);
      const float hi = __uint_as_float(w & 0xffff0000u) * (i < 2 ? s0[2 * i + 1] : s1[2 * i - 3]);
      amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(lo), __builtin_fabsf(hi)));
    }
  }
  amax = wave_max(amax);
  if (lane == 0) sx[t] = amax / 127.0f;
  const float rr = amax > 0.0f ? 127.0f / amax : 0.0f;
  int8_t *qr = qx + t * H;
  for (int c = lane; c < nchunk; c += 64) {
    const v4i raw = *reinterpret_cast<const v4i *>(xr + c * 8);
    const v4f s0 = *reinterpret_cast<const v4f *>(inv_s + c * 8);
    const v4f s1 = *reinterpret_cast<const v4f *>(inv_s + c * 8 + 4);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = (uint32_t)raw[i];
      const float lo = __uint_as_float(w << 16) * (i < 2 ? s0[2 * i] : s1[2 * i - 4]);
      const float hi = __uint_as_float(w & 0xffff0000u) * (i < 2 ? s0[2 * i + 1] : s1[2 * i - 3]);
      const uint32_t qlo = (uint32_t)(q8(lo, rr) & 0xff), qhi = (uint32_t)(q8(hi, rr) & 0xff);
      packed[i >> 1] |= (qlo | (qhi << 8)) << (16 * (i & 1));
    }
    *reinterpret_cast<uint2 *>(qr + c * 8) = make_uint2(packed[0], packed[1]);
  }
}

// h fp32 [A][F] with row max |h| in amax (float bits) -> qh int8, sh fp32.
// Rows past the number of kept rows (offsets[E]) are left alone.
__global__ __launch_bounds__(256) void requant_kernel(const float *__restrict__ h,
                                                      const uint32_t *__restrict__ amax_bits,
                                                      const int32_t *__restrict__ offsets, int E,
                                                      int F, int8_t *__restrict__ qh,
                                                      float *__restrict__ sh) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= offsets[E]) return;
  const float amax = __uint_as_float(amax_bits[r]);
  if (lane == 0) sh[r] = amax / 127.0f;
  const float rr = amax > 0.0f ? 127.0f / amax : 0.0f;
  const float *hr = h + r * F;
  int8_t *qr = qh + r * F;
  for (int c = lane; c < (F >> 2); c += 64) {
    const v4f v = *reinterpret_cast<const v4f *>(hr + c * 4);
    const uint32_t p = (uint32_t)(q8(v[0], rr) & 0xff) | ((uint32_t)(q8(v[1], rr) & 0xff) << 8) |
                       ((uint32_t)(q8(v[2], rr) & 0xff) << 16) |
                       ((uint32_t)(q8(v[3], rr) & 0xff) << 24);
    *reinterpret_cast<uint32_t *>(qr + c * 4) = p;
  }
}

}  // namespace

hipError_t launch_act_quant(const uint16_t *x, const float *inv_s, int64_t T, int H, int8_t *qx,
                            float *sx, hipStream_t st) {
  act_quant_kernel<<<dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st>>>(x, inv_s, T, H, qx, sx);
  return hipGetLastError();
}

hipError_t launch_requant(const float *h, const uint32_t *amax, const int32_t *offsets, int E,
                          int64_t A, int F, int8_t *qh, float *sh, hipStream_t st) {
  requant_kernel<<<dim3((unsigned)((A + 3) / 4)), dim3(256), 0, st>>>(h, amax, offsets, E, F, qh,
                                                                       sh);
  return hipGetLastError();
}

}  // namespace moe
