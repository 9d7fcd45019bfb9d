// gemm_stream.hip -- grouped INT8 GEMMs for few rows per expert (decode).
//
// "MiniMax-M3 W8A8 inference on K100AI" (mhpq.cn/news/1068415) §1.1: decode
// is bound by reading expert weights, and W8A8 halves those bytes (§1.3);
// §4.3: one kernel runs a whole batch of experts instead of many small GEMMs.
// Here every block streams one panel of one expert's fragment-tiled weights
// exactly once, from HBM, as contiguous 1 KB wavefront loads, and multiplies
// it with all rows routed to that expert (INT8 x INT8 -> INT32 on
// v_mfma_i32_16x16x64_i8). The weight panel is the MFMA A operand (16 output
// channels), the token rows the B operand (16 rows per tile), so the few
// rows of a decode step cost no extra weight traffic.
//
// Grid (panels, E); block = 4 wavefronts splitting K; partial INT32 sums are
// reduced exactly through LDS, then the epilogue:
//   GEMM1 (gate/up, K = H): g = acc_g*sx*s_g, u = acc_u*sx*s_u,
//         h = silu(g)*u (fp32) -> h[row][f]; row max |h| -> amax (atomic max
//         on the float bits, order independent);
//   GEMM2 (down, K = F):    y[row][n] = acc*sh*s_d[n] (fp32).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRT = 2;  // row tiles of 16 held per pass (32 rows)

// kGateUp: GEMM1 (panel pair gate p / up F/16+p). Otherwise GEMM2 with NP
// consecutive output panels per block.
template <bool kGateUp, int NP>
__global__ __launch_bounds__(256) void gemm_stream_kernel(
    const int8_t *__restrict__ act, const float *__restrict__ act_scale,
    const int32_t *__restrict__ sorted, int k, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, const int8_t *__restrict__ w,
    const float *__restrict__ wscale, int K, int F, int H, float *__restrict__ out,
    uint32_t *__restrict__ amax, int32_t *__restrict__ acc1_dbg) {
  constexpr int NA = kGateUp ? 2 : NP;  // A panels per k tile
  const int e = blockIdx.y;
  const int p = blockIdx.x;
  const int R = counts[e];
  if (R == 0) return;
  const int row0 = offsets[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int KT = K >> 6;
  const int kt0 = (wave * KT) >> 2, kt1 = ((wave + 1) * KT) >> 2;
  const int N = kGateUp ? 2 * F : H;  // rows of the expert's weight matrix
  const int8_t *wexp = w + (size_t)e * (size_t)N * (size_t)K;
  const int8_t *wp[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const int nt = kGateUp ? (a == 0 ? p : (F >> 4) + p) : p * NP + a;
    wp[a] = wexp + frag_tile(nt, 0, K) + lane * 16;
  }
  __shared__ v4i red[4][NA * kRT][64];

  for (int base = 0; base < R; base += 16 * kRT) {
    const int8_t *bp[kRT];
    bool bv[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const int r = base + rt * 16 + (lane & 15);
      bv[rt] = r < R;
      size_t arow = 0;
      if (bv[rt]) arow = kGateUp ? (size_t)(sorted[row0 + r] / k) : (size_t)(row0 + r);
      bp[rt] = act + arow * (size_t)K + (lane >> 4) * 16;
    }
    v4i acc[NA][kRT];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) acc[a][rt] = v4i{0, 0, 0, 0};
#pragma unroll 4
    for (int kt = kt0; kt < kt1; ++kt) {
      v4i af[NA], bf[kRT];
#pragma unroll
      for (int a = 0; a < NA; ++a)
        af[a] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(wp[a] + ((size_t)kt << 10)));
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        bf[rt] = bv[rt] ? *reinterpret_cast<const v4i *>(bp[rt] + kt * 64) : v4i{0, 0, 0, 0};
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) acc[a][rt] = mfma16(af[a], bf[rt], acc[a][rt]);
    }
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) red[wave][a * kRT + rt][lane] = acc[a][rt];
    __syncthreads();
    // Epilogue: combination c = (panel group, row tile) handled by wave c % 4.
    constexpr int NC = (kGateUp ? 1 : NP) * kRT;
    for (int c = wave; c < NC; c += 4) {
      const int rt = c % kRT, pg = c / kRT;
      const int r = base + rt * 16 + (lane & 15);
      const bool valid = r < R;
      const int ch0 = (lane >> 4) * 4;  // first of this lane's 4 output channels
      if (kGateUp) {
        v4i g = red[0][rt][lane], u = red[0][kRT + rt][lane];
#pragma unroll
        for (int wv = 1; wv < 4; ++wv) {
          g += red[wv][rt][lane];
          u += red[wv][kRT + rt][lane];
        }
        float hmax = 0.0f;
        if (valid) {
          const int row = row0 + r;
          const int t = sorted[row] / k;
          const float sxv = act_scale[t];
          const int f0 = p * 16 + ch0;
          const float *sg = wscale + (size_t)e * 2 * F + f0;
          const float *su = sg + F;
          v4f hv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gv = (float)g[i] * sxv * sg[i];
            const float uv = (float)u[i] * sxv * su[i];
            hv[i] = gv / (1.0f + expf(-gv)) * uv;
            hmax = __builtin_fmaxf(hmax, __builtin_fabsf(hv[i]));
          }
          *reinterpret_cast<v4f *>(out + (size_t)row * F + f0) = hv;
          if (acc1_dbg) {
            *reinterpret_cast<v4i *>(acc1_dbg + (size_t)row * 2 * F + f0) = g;
            *reinterpret_cast<v4i *>(acc1_dbg + (size_t)row * 2 * F + F + f0) = u;
          }
        }
        hmax = __builtin_fmaxf(hmax, __shfl_xor(hmax, 16, 64));
        hmax = __builtin_fmaxf(hmax, __shfl_xor(hmax, 32, 64));
        if (valid && lane < 16) atomicMax(amax + row0 + r, __float_as_uint(hmax));
      } else {
        v4i s = red[0][pg * kRT + rt][lane];
#pragma unroll
        for (int wv = 1; wv < 4; ++wv) s += red[wv][pg * kRT + rt][lane];
        if (valid) {
          const int row = row0 + r;
          const float shv = act_scale[row];
          const int n0 = (p * NP + pg) * 16 + ch0;
          const float *sd = wscale + (size_t)e * H + n0;
          v4f yv;
#pragma unroll
          for (int i = 0; i < 4; ++i) yv[i] = (float)s[i] * shv * sd[i];
          *reinterpret_cast<v4f *>(out + (size_t)row * H + n0) = yv;
        }
      }
    }
    __syncthreads();
  }
}

constexpr int kDownPanels = 4;

}  // namespace

hipError_t launch_gemm1_stream(const int8_t *qx, const float *sx, const int32_t *sorted, int k,
                               const int32_t *counts, const int32_t *offsets, const int8_t *w_gu,
                               const float *s_gu, int H, int F, int E, float *h, uint32_t *amax,
                               int32_t *acc1_dbg, hipStream_t st) {
  dim3 grid((unsigned)(F / 16), (unsigned)E);
  gemm_stream_kernel<true, 1><<<grid, dim3(256), 0, st>>>(qx, sx, sorted, k, counts, offsets, w_gu,
                                                          s_gu, H, F, H, h, amax, acc1_dbg);
  return hipGetLastError();
}

hipError_t launch_gemm2_stream(const int8_t *qh, const float *sh, const int32_t *counts,
                               const int32_t *offsets, const int8_t *w_d, const float *s_d, int H,
                               int F, int E, float *y, hipStream_t st) {
  dim3 grid((unsigned)(H / (16 * kDownPanels)), (unsigned)E);
  gemm_stream_kernel<false, kDownPanels><<<grid, dim3(256), 0, st>>>(
      qh, sh, nullptr, 1, counts, offsets, w_d, s_d, F, F, H, y, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace moe
