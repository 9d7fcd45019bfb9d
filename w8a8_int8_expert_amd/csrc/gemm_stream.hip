// gemm_stream.hip -- grouped INT8 GEMMs for few rows per expert (decode).
//
// "MiniMax-M3 W8A8 inference on K100AI" (mhpq.cn/news/1068415) §1.1: decode
// is bound by reading expert weights, and W8A8 halves those bytes (§1.3);
// §4.3: one kernel runs a whole batch of experts instead of many small GEMMs,
// and the matmuls stay in INT8 with no dequantise between them.
// Every block streams one panel of one expert's fragment-tiled weights
// exactly once, from HBM, as contiguous 1 KB wavefront loads, and multiplies
// it with all rows routed to that expert (INT8 x INT8 -> INT32 on
// v_mfma_i32_16x16x64_i8; FP8 codes: -> fp32 on the 16x16x128 FP8
// instruction, "超大规模模型推理的Day0适配实践" §二.1 and §四). The weight panel is the MFMA A operand (16 output
// channels), the token rows the B operand (16 rows per tile), so the few
// rows of a decode step cost no extra weight traffic.
//
// Block = 4 wavefronts = (4/KS) panel groups x KS K-splits. A group owns NPW
// panel units (GEMM1 unit: the 16 gate rows f..f+15 and the matching 16 up
// rows; GEMM2 unit: 16 output channels); its KS wavefronts take the 1 KB
// k-tiles ks, ks+KS, ks+2KS, ... so that at any moment the block reads
// adjacent tiles of each panel. With KS > 1 the partial INT32 sums are
// reduced exactly through LDS. Grid (units / ((4/KS)*NPW), E). Epilogue:
//   GEMM1 (gate/up, K = H): g = acc_g*sx*s_g, u = acc_u*sx*s_u,
//         h = silu(g)*u (fp32) -> h[row][f]; row max |h| -> amax (atomic max
//         on the float bits, order independent);
//   GEMM2 (down, K = F):    y[row][n] = acc*sh*s_d[n] (fp32).
// Requantisation and combine are launches of their own: handing a unit of
// work to its last-finishing block needs a device-scope release per block,
// which writes back the XCD's L2 and cost more than the launches it saved.
#include "layer_device.h"

namespace moe {
namespace {

constexpr int kRT = 2;  // row tiles of 16 held per pass (32 rows)

struct StreamArgs {
  const int8_t *act;        // GEMM1: qx [T][H] by token; GEMM2: qh fragment-tiled by row
  const float *act_scale;   // GEMM1: sx [T];    GEMM2: sh [rows]
  const int32_t *sorted;    // GEMM1 only
  int k;
  const int32_t *counts, *offsets;  // offsets: padded (16-row aligned) group starts
  const int32_t *dense_off;         // GEMM1: dense group starts (debug rows)
  const int8_t *w;          // fragment-tiled weights
  const float *wscale;
  int K, F, H;
  float *out;               // GEMM1: h [A][F]; GEMM2: y [A][H]
  uint32_t *amax;           // GEMM1 only
  int32_t *acc1_dbg;        // GEMM1 only, may be NULL; dense rows
};

// Accumulators: INT32 for INT8 codes, fp32 for FP8 codes.
template <bool kF8> struct Acc16 { typedef v4i T; };
template <> struct Acc16<true> { typedef v4f T; };

template <bool kGateUp, int NPW, int KS, int U, bool kF8>
__global__ __launch_bounds__(256) void gemm_stream_kernel(const StreamArgs a) {
  typedef typename Acc16<kF8>::T Acc;
  static_assert(!kF8 || U % 2 == 0, "FP8 pairs k-tiles");
  constexpr int NA = kGateUp ? 2 * NPW : NPW;  // weight panels per group
  constexpr int NG = 4 / KS;                   // panel groups per block
  const int e = blockIdx.y;
  const int R = a.counts[e];
  if (R == 0) return;
  const int row0 = a.offsets[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave / KS, ks = wave % KS;
  const int K = a.K, F = a.F, H = a.H;
  const int KT = K >> 6;
  const int u0 = (blockIdx.x * NG + grp) * NPW;  // first panel unit of this group
  const int N = kGateUp ? 2 * F : H;             // rows of the expert's weight matrix
  const int8_t *wexp = a.w + (size_t)e * (size_t)N * (size_t)K;
  const int8_t *wp[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int nt = kGateUp ? (i < NPW ? u0 + i : (F >> 4) + u0 + i - NPW) : u0 + i;
    wp[i] = wexp + frag_tile(nt, 0, K) + lane * 16;
  }
  __shared__ Acc red[KS > 1 ? 4 : 1][KS > 1 ? NA * kRT : 1][64];

  for (int base = 0; base < R; base += 16 * kRT) {
    const int8_t *bp[kRT];
    bool bv[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const int r = base + rt * 16 + (lane & 15);
      bv[rt] = r < R;
      if (kGateUp) {
        const size_t tok = bv[rt] ? (size_t)(a.sorted[row0 + r] / a.k) : 0;
        bp[rt] = a.act + tok * (size_t)K + (lane >> 4) * 16;
      } else {
        // Row tile (row0 + base)/16 + rt of the tiled operand: lane l holds
        // row l%16 of it, exactly the operand order below.
        bp[rt] = a.act + frag_tile(((row0 + base) >> 4) + rt, 0, K) + lane * 16;
      }
    }
    const int astep = kGateUp ? 64 : 1024;  // bytes per k tile of the operand row
    Acc acc[NA][kRT];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) acc[i][rt] = Acc{0, 0, 0, 0};
    // This wavefront's k-tiles, U at a time: all loads of a batch are issued
    // before its MFMAs, so U*NA weight tiles are in flight per wavefront.
    const int nk = (KT - ks + KS - 1) / KS;
    auto load = [&](int it, v4i *af, v4i *bf) {
      const int kt = ks + it * KS;
#pragma unroll
      for (int i = 0; i < NA; ++i)
        af[i] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(wp[i] + ((size_t)kt << 10)));
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        bf[rt] = bv[rt] ? *reinterpret_cast<const v4i *>(bp[rt] + (size_t)kt * astep)
                        : v4i{0, 0, 0, 0};
    };
    // INT8: one k-tile per v_mfma_i32_16x16x64_i8. FP8: two k-tiles per
    // v_mfma_scale_f32_16x16x128_f8f6f4 (a lone last tile is paired with zeros).
    auto mma = [&](const v4i *af, const v4i *bf, const v4i *af2, const v4i *bf2) {
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          if constexpr (kF8)
            acc[i][rt] = mfma16f8(af[i], af2[i], bf[rt], bf2[rt], acc[i][rt]);
          else
            acc[i][rt] = mfma16(af[i], bf[rt], acc[i][rt]);
        }
    };
    int it = 0;
    for (; it + U <= nk; it += U) {
      v4i af[U][NA], bf[U][kRT];
#pragma unroll
      for (int u = 0; u < U; ++u) load(it + u, af[u], bf[u]);
#pragma unroll
      for (int u = 0; u < U; u += kF8 ? 2 : 1) mma(af[u], bf[u], af[u + (kF8 ? 1 : 0)], bf[u + (kF8 ? 1 : 0)]);
    }
    for (; it < nk; ++it) {
      v4i af[NA], bf[kRT], z[NA > kRT ? NA : kRT];
#pragma unroll
      for (int i = 0; i < (NA > kRT ? NA : kRT); ++i) z[i] = v4i{0, 0, 0, 0};
      load(it, af, bf);
      mma(af, bf, z, z);
    }
    if (KS > 1) {
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) red[wave][i * kRT + rt][lane] = acc[i][rt];
      __syncthreads();
    }
    // Epilogue: combination c = (unit q, row tile rt) of the group, taken by
    // its wavefront ks == c % KS. Lane holds row base + rt*16 + (lane & 15)
    // and the 4 output channels ch0..ch0+3 of the unit, ch0 = (lane >> 4)*4.
    const int ch0 = (lane >> 4) * 4;
#pragma unroll
    for (int c = 0; c < NPW * kRT; ++c) {
      if (c % KS != ks) continue;
      const int q = c / kRT, rt = c % kRT;
      const int r = base + rt * 16 + (lane & 15);
      const bool valid = r < R;
      const int row = row0 + r;
      auto total = [&](int i) -> Acc {
        if (KS == 1) return acc[i][rt];
        Acc sum = red[grp * KS][i * kRT + rt][lane];
#pragma unroll
        for (int w = 1; w < KS; ++w) sum += red[grp * KS + w][i * kRT + rt][lane];
        return sum;
      };
      if (kGateUp) {
        float hmax = 0.0f;
        const Acc g = total(q), u = total(NPW + q);
        if (valid) {
          const float sxv = a.act_scale[a.sorted[row] / a.k];
          const int f0 = (u0 + q) * 16 + ch0;
          const float *sg = a.wscale + (size_t)e * 2 * F + f0;
          const float *su = sg + F;
          v4f hv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gv = (float)g[i] * sxv * sg[i];
            const float uv = (float)u[i] * sxv * su[i];
            hv[i] = gv / (1.0f + expf(-gv)) * uv;
            hmax = __builtin_fmaxf(hmax, __builtin_fabsf(hv[i]));
          }
          *reinterpret_cast<v4f *>(a.out + (size_t)row * F + f0) = hv;
          if (a.acc1_dbg) {
            const size_t drow = (size_t)(a.dense_off[e] + r);
            *reinterpret_cast<v4i *>(a.acc1_dbg + drow * 2 * F + f0) = __builtin_bit_cast(v4i, g);
            *reinterpret_cast<v4i *>(a.acc1_dbg + drow * 2 * F + F + f0) =
                __builtin_bit_cast(v4i, u);
          }
        }
        hmax = __builtin_fmaxf(hmax, __shfl_xor(hmax, 16, 64));
        hmax = __builtin_fmaxf(hmax, __shfl_xor(hmax, 32, 64));
        if (valid && lane < 16) atomicMax(a.amax + row, __float_as_uint(hmax));
      } else {
        const Acc sacc = total(q);
        if (valid) {
          const float shv = a.act_scale[row];
          const int n0 = (u0 + q) * 16 + ch0;
          const float *sd = a.wscale + (size_t)e * H + n0;
          v4f yv;
#pragma unroll
          for (int i = 0; i < 4; ++i) yv[i] = (float)sacc[i] * shv * sd[i];
          *reinterpret_cast<v4f *>(a.out + (size_t)row * H + n0) = yv;
        }
      }
    }
    if (KS > 1) __syncthreads();
  }
}

// Shapes chosen by timing the decode step (hidden 4096, FFN 1536, 64
// experts, ~4 rows each) on MI355X: GEMM1 streams 2 gate + 2 up panels per
// block (256 KB), GEMM2 2 panels (48 KB); both split K over the 4 waves.
// FP8 GEMM2 takes its 6 k-tiles per wave in one batch (with 4, the last two
// ran one at a time: 70 against 65.5 us).
constexpr int kNpwGateUp = 2, kKsGateUp = 4, kUGateUp = 2;
constexpr int kNpwDown = 2, kKsDown = 4, kUDown = 4, kUDownF8 = 6;

}  // namespace

hipError_t launch_gemm1_stream(const int8_t *qx, const float *sx, const int32_t *sorted, int k,
                               const int32_t *counts, const int32_t *offsets,
                               const int32_t *dense_off, const int8_t *w_gu, const float *s_gu,
                               int H, int F, int E, float *h, uint32_t *amax, int32_t *acc1_dbg,
                               bool fp8, hipStream_t st, Timing tm) {
  StreamArgs a{};
  a.act = qx; a.act_scale = sx; a.sorted = sorted; a.k = k; a.counts = counts;
  a.offsets = offsets; a.dense_off = dense_off; a.w = w_gu; a.wscale = s_gu; a.K = H; a.F = F; a.H = H;
  a.out = h; a.amax = amax; a.acc1_dbg = acc1_dbg;
  const dim3 grid((unsigned)(F / (16 * (4 / kKsGateUp) * kNpwGateUp)), (unsigned)E);
  if (fp8)
    return launch_kernel(gemm_stream_kernel<true, kNpwGateUp, kKsGateUp, kUGateUp, true>, grid,
                         dim3(256), st, tm, a);
  return launch_kernel(gemm_stream_kernel<true, kNpwGateUp, kKsGateUp, kUGateUp, false>, grid,
                       dim3(256), st, tm, a);
}

hipError_t launch_gemm2_stream(const int8_t *qh, const float *sh, const int32_t *counts,
                               const int32_t *offsets, const int8_t *w_d, const float *s_d, int H,
                               int F, int E, float *y, bool fp8, hipStream_t st, Timing tm) {
  StreamArgs a{};
  a.act = qh; a.act_scale = sh; a.k = 1; a.counts = counts; a.offsets = offsets; a.w = w_d;
  a.wscale = s_d; a.K = F; a.F = F; a.H = H; a.out = y;
  const dim3 grid((unsigned)(H / (16 * (4 / kKsDown) * kNpwDown)), (unsigned)E);
  if (fp8)
    return launch_kernel(gemm_stream_kernel<false, kNpwDown, kKsDown, kUDownF8, true>, grid,
                         dim3(256), st, tm, a);
  return launch_kernel(gemm_stream_kernel<false, kNpwDown, kKsDown, kUDown, false>, grid,
                       dim3(256), st, tm, a);
}

}  // namespace moe
