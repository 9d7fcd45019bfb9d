// calibrate.hip -- SmoothQuant calibration and per-channel weight quantisation.
//
// "MiniMax-M3 W8A8 inference on K100AI" (mhpq.cn/news/1068415) §3.2: W8A8
// with per-channel weights, per-token activations and SmoothQuant (alpha sets
// how much of the activation range moves into the weights); §1.2: weight
// ranges come from per-channel statistics. SmoothQuant's published scale is
//   s_j = max|X_j|^alpha / max|W_j|^(1-alpha)
// with X' = X/s and W' = W*s along input channel j. One s[H] serves the whole
// layer (every expert's gate and up projections read the same token), so
// max|W_j| runs over all experts and both projections; the down projection
// is not smoothed. Launch order: clear + column maxima, scales, quantisation.
#include "moe_internal.h"

namespace moe {
namespace {

// ax[j] = max_n |calib_x[n][j]|  (one thread per column; float bits).
__global__ __launch_bounds__(256) void colmax_x_kernel(const uint16_t *__restrict__ x,
                                                       int64_t n, int H, uint32_t *__restrict__ ax,
                                                       uint32_t *__restrict__ aw) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= H) return;
  float m = 0.0f;
  for (int64_t r = 0; r < n; ++r) m = __builtin_fmaxf(m, __builtin_fabsf(bf16_to_f32(x[r * H + j])));
  ax[j] = __float_as_uint(m);
  aw[j] = 0u;  // cleared here, filled by colmax_w_kernel
}

// aw[j] = max over rows of W_gate and W_up ([E*F][H] each) of |W[r][j]|.
// Grid (H/256, row chunks); partial maxima merged with atomicMax on the
// float bits of non-negative values (order independent).
__global__ __launch_bounds__(256) void colmax_w_kernel(const float *__restrict__ wg,
                                                       const float *__restrict__ wu, int64_t rows,
                                                       int64_t rows_per_chunk, int H,
                                                       uint32_t *__restrict__ aw) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= H) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
  const int64_t r1 = r0 + rows_per_chunk < rows ? r0 + rows_per_chunk : rows;
  float m = 0.0f;
  for (int64_t r = r0; r < r1; ++r) {
    m = __builtin_fmaxf(m, __builtin_fabsf(wg[r * H + j]));
    m = __builtin_fmaxf(m, __builtin_fabsf(wu[r * H + j]));
  }
  atomicMax(aw + j, __float_as_uint(m));
}

// s_j in fp64, rounded once to fp32; s_j = 1 for an empty range.
__global__ __launch_bounds__(256) void smooth_kernel(const uint32_t *__restrict__ ax,
                                                     const uint32_t *__restrict__ aw, float alpha,
                                                     int H, float *__restrict__ s,
                                                     float *__restrict__ inv_s) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= H) return;
  const float a = __uint_as_float(ax[j]), b = __uint_as_float(aw[j]);
  float sj = 1.0f;
  if (a > 0.0f && b > 0.0f) {
    const double al = (double)alpha;
    sj = (float)(pow((double)a, al) / pow((double)b, 1.0 - al));
  }
  s[j] = sj;
  inv_s[j] = 1.0f / sj;
}

// One wavefront per output row. Row r < E*2F is a gate/up row of the
// smoothed [E][2F][H] matrix; otherwise a down row of [E][H][F]. The row's
// codes are written into the fragment-tiled layout: the 16 consecutive
// input channels k..k+15 (k % 16 == 0) of row n are 16 contiguous bytes at
// tile (n/16, k/64) + (((k%64)/16)*16 + n%16)*16.
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const float *__restrict__ wg, const float *__restrict__ wu, const float *__restrict__ wd,
    const float *__restrict__ s, int H, int F, int E, int8_t *__restrict__ w_gu,
    float *__restrict__ s_gu, int8_t *__restrict__ w_d, float *__restrict__ s_d, bool fp8) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t n_gu = (int64_t)E * 2 * F;
  if (r >= n_gu + (int64_t)E * H) return;
  const bool gu = r < n_gu;
  const float *src;
  int K, n, N;
  int64_t e;
  int8_t *dst;
  float *scale;
  if (gu) {
    e = r / (2 * F);
    n = (int)(r % (2 * F));
    src = n < F ? wg + (e * F + n) * (int64_t)H : wu + (e * F + (n - F)) * (int64_t)H;
    K = H; N = 2 * F;
    dst = w_gu + e * (int64_t)N * K;
    scale = s_gu + r;
  } else {
    const int64_t rd = r - n_gu;
    e = rd / H;
    n = (int)(rd % H);
    src = wd + rd * (int64_t)F;
    K = F; N = H;
    dst = w_d + e * (int64_t)N * K;
    scale = s_d + rd;
  }
  float amax = 0.0f;
  for (int c = lane; c < (K >> 4); c += 64) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = src[c * 16 + i];
      if (gu) v = v * s[c * 16 + i];
      amax = __builtin_fmaxf(amax, __builtin_fabsf(v));
    }
  }
  amax = wave_max(amax);
  const float qmax = fp8 ? kFp8Max : 127.0f;
  if (lane == 0) *scale = amax / qmax;
  const float rr = amax > 0.0f ? qmax / amax : 0.0f;
  for (int c = lane; c < (K >> 4); c += 64) {
    const int kk = c * 16;
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = src[kk + 4 * i + j];
        if (gu) v[j] = v[j] * s[kk + 4 * i + j];
      }
      p[i] = codes4(v, rr, fp8);
    }
    int8_t *d = dst + frag_tile(n >> 4, kk >> 6, K) + ((((kk & 63) >> 4) << 4) + (n & 15)) * 16;
    *reinterpret_cast<v4i *>(d) = v4i{(int)p[0], (int)p[1], (int)p[2], (int)p[3]};
  }
}

}  // namespace

hipError_t launch_calib_colmax(const uint16_t *calib_x, int64_t n_calib, const float *w_gate,
                               const float *w_up, int H, int F, int E, uint32_t *ax, uint32_t *aw,
                               hipStream_t st) {
  const unsigned cb = (unsigned)((H + 255) / 256);
  const hipError_t err =
      launch_kernel(colmax_x_kernel, dim3(cb), dim3(256), st, Timing{}, calib_x, n_calib, H, ax, aw);
  if (err != hipSuccess) return err;
  const int64_t rows = (int64_t)E * F;
  const int64_t chunks = rows < 512 ? rows : 512;
  const int64_t per = (rows + chunks - 1) / chunks;
  return launch_kernel(colmax_w_kernel, dim3(cb, (unsigned)((rows + per - 1) / per)), dim3(256),
                       st, Timing{}, w_gate, w_up, rows, per, H, aw);
}

// Static clipping threshold ("一晚上完成MoE模型推理优化…" §3.2: calibration
// clips the activations at a percentile of their range): the m-th largest of
// the N = n_calib * H values |fl32(x[n][j] * inv_s[j])|, m = N - r + 1 for the
// percentile's rank r. One block decides the answer bit by bit from the top
// (non-negative floats order as unsigned integers): a bit is kept when at
// least m values are >= the answer with it set. N = 0 writes 0 (no clip).
__global__ __launch_bounds__(1024) void clip_threshold_kernel(const uint16_t *__restrict__ x,
                                                              int64_t n_calib, int H,
                                                              const float *__restrict__ inv_s,
                                                              int64_t m, float *__restrict__ out) {
  __shared__ long long wcnt[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t N = n_calib * H;
  uint32_t ans = 0u;
  for (int bit = 30; bit >= 0 && N > 0; --bit) {
    const uint32_t cand = ans | (1u << bit);
    long long cnt = 0;
    for (int j = tid; j < H; j += 1024) {
      const float sj = inv_s[j];
      for (int64_t n = 0; n < n_calib; ++n) {
        const float v = __uint_as_float((uint32_t)x[n * H + j] << 16) * sj;
        cnt += __float_as_uint(__builtin_fabsf(v)) >= cand ? 1 : 0;
      }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) cnt += __shfl_xor(cnt, o, 64);
    if (lane == 0) wcnt[wave] = cnt;
    __syncthreads();
    long long total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) total += wcnt[w];
    __syncthreads();
    if (total >= m) ans = cand;
  }
  if (tid == 0) *out = __uint_as_float(ans);
}

hipError_t launch_calib_clip(const uint16_t *calib_x, int64_t n_calib, int H, const float *inv_s,
                             int64_t m, float *out, hipStream_t st) {
  return launch_kernel(clip_threshold_kernel, dim3(1), dim3(1024), st, Timing{}, calib_x, n_calib,
                       H, inv_s, m, out);
}

hipError_t launch_calib_smooth(const uint32_t *ax, const uint32_t *aw, float alpha, int H,
                               float *s, float *inv_s, hipStream_t st) {
  return launch_kernel(smooth_kernel, dim3((unsigned)((H + 255) / 256)), dim3(256), st, Timing{},
                       ax, aw, alpha, H, s, inv_s);
}

hipError_t launch_calib_quant(const float *w_gate, const float *w_up, const float *w_down,
                              const float *s, int H, int F, int E, int8_t *w_gu, float *s_gu,
                              int8_t *w_d, float *s_d, bool fp8, hipStream_t st) {
  const int64_t rows = (int64_t)E * 2 * F + (int64_t)E * H;
  return launch_kernel(quant_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), st, Timing{},
                       w_gate, w_up, w_down, s, H, F, E, w_gu, s_gu, w_d, s_d, fp8);
}

}  // namespace moe
