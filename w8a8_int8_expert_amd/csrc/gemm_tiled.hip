// gemm_tiled.hip -- grouped INT8 GEMMs for many rows per expert (prefill).
//
// "MiniMax-M3 W8A8 inference on K100AI" (mhpq.cn/news/1068415) §1.1/§4.3:
// batch-level scheduling so that expert compute is one large grouped GEMM
// rather than many small ones; §1.2: INT8 x INT8 with integer accumulation,
// dequantised afterwards; "一晚上完成MoE模型推理优化…" §4.1: the activation
// that follows a linear layer is fused into it (SwiGLU in GEMM1's epilogue).
//
// One block computes a 128-row x 256-column tile of one expert on
// v_mfma_i32_32x32x32_i8:
//   rows    = 128 consecutive permuted rows of the expert (the M tile);
//   columns = GEMM1: 128 gate rows and the matching 128 up rows of the
//             expert's [2F][H] weights (wave w owns gate/up columns
//             f0+32w..f0+32w+31, so g and u of one h element meet in the
//             same lane); GEMM2: 256 output channels (64 per wave).
// Activations (GEMM1: gathered rows of qx; GEMM2: contiguous rows of qh) are
// staged through LDS, double buffered, in an XOR-swizzled layout that makes
// the 16-byte fragment reads conflict free. Weight fragments come straight
// from the fragment-tiled layout into registers (each wave owns its columns,
// so they are not shared and need no LDS).
// M tiles of all experts are numbered consecutively (mtile_off, written by
// the scan kernel); blocks past the last tile exit at once. Blocks are
// renumbered so that each XCD (one L2) works on a contiguous range of tiles.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = kTiledBM;   // 128
constexpr int BK = 64;         // K per step (one fragment tile column)

__device__ __forceinline__ int lds_a_off(int m, int seg) {
  return m * BK + ((seg ^ ((m >> 2) & 3)) << 4);
}

template <bool kGateUp>
__global__ __launch_bounds__(256, 2) void gemm_tiled_kernel(
    const int8_t *__restrict__ act, const float *__restrict__ act_scale,
    const int32_t *__restrict__ sorted, int k, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ mtile_off, int E,
    const int8_t *__restrict__ w, const float *__restrict__ wscale, int K, int F, int H,
    void *__restrict__ out_v, uint32_t *__restrict__ amax, int32_t *__restrict__ acc1_dbg) {
  __shared__ __attribute__((aligned(16))) int8_t lds_a[2][BM * BK];
  __shared__ float row_scale[BM];
  __shared__ int32_t row_tok[BM];

  // XCD-aware renumbering of the linear block id, then (m tile, n tile).
  const int nbx = gridDim.x, nby = gridDim.y;
  const int nb = nbx * nby;
  const int b = blockIdx.x + nbx * blockIdx.y;
  const int xcd = b & 7, idx = b >> 3, q = nb >> 3, rem = nb & 7;
  const int logical = xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
  const int mt = logical % nbx;   // global M tile (x: M tiles)
  const int ntile = logical / nbx;

  if (mt >= mtile_off[E]) return;
  int lo = 0, hi = E;  // largest e with mtile_off[e] <= mt
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mtile_off[mid] <= mt) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int R = counts[e];
  const int row0 = offsets[e];
  const int m0 = (mt - mtile_off[e]) * BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = kGateUp ? 2 * F : H;
  const int KT = K / BK;

  // Row bookkeeping: token (GEMM1) and activation scale of each tile row.
  if (tid < BM) {
    const int r = m0 + tid;
    int tok = -1;
    float sc = 0.0f;
    if (r < R) {
      const int row = row0 + r;
      tok = kGateUp ? sorted[row] / k : row;
      sc = act_scale[tok];
    }
    row_tok[tid] = tok;
    row_scale[tid] = sc;
  }
  __syncthreads();

  // Global -> LDS assignment: thread owns 16-byte chunks (row, seg) for rows
  // tid>>2 and 64 + (tid>>2), segment tid&3.
  const int seg = tid & 3;
  const int8_t *asrc[2];
  bool aval[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = (tid >> 2) + 64 * i;
    const int tok = row_tok[m];
    aval[i] = tok >= 0;
    asrc[i] = act + (size_t)(tok >= 0 ? tok : 0) * (size_t)K + seg * 16;
  }

  // Weight fragment pointers: column tile ct of this wave.
  const int8_t *wexp = w + (size_t)e * (size_t)N * (size_t)K;
  const int8_t *bsrc[2];
  int ncol[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    int nc0;
    if (kGateUp) nc0 = (ct == 0 ? 0 : F) + ntile * 128 + wave * 32;
    else nc0 = ntile * 256 + wave * 64 + ct * 32;
    const int n = nc0 + (lane & 31);
    ncol[ct] = n;
    bsrc[ct] = wexp + frag_tile(n >> 4, 0, K) + ((((lane >> 5) << 4) + (n & 15)) << 4);
  }

  v16i acc[4][2];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rt][ct][i] = 0;

  // Prologue: stage k tile 0.
  v4i anext[2], bcur[2][2], bnext[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    anext[i] = aval[i] ? *reinterpret_cast<const v4i *>(asrc[i]) : v4i{0, 0, 0, 0};
    *reinterpret_cast<v4i *>(&lds_a[0][lds_a_off((tid >> 2) + 64 * i, seg)]) = anext[i];
  }
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      bcur[ct][hf] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(bsrc[ct] + hf * 512));
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        anext[i] = aval[i] ? *reinterpret_cast<const v4i *>(asrc[i] + (size_t)(kt + 1) * BK)
                           : v4i{0, 0, 0, 0};
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          bnext[ct][hf] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(
              bsrc[ct] + ((size_t)(kt + 1) << 10) + hf * 512));
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int m = rt * 32 + (lane & 31);
      v4i afr[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        afr[hf] = *reinterpret_cast<const v4i *>(&lds_a[cur][lds_a_off(m, 2 * hf + (lane >> 5))]);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) acc[rt][ct] = mfma32(afr[hf], bcur[ct][hf], acc[rt][ct]);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<v4i *>(&lds_a[cur ^ 1][lds_a_off((tid >> 2) + 64 * i, seg)]) = anext[i];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) bcur[ct][hf] = bnext[ct][hf];
    }
    __syncthreads();
  }

  // Epilogue. Lane holds column (lane & 31) of each 32x32 tile and rows
  // rt*32 + (i/4)*8 + (lane/32)*4 + i%4, i < 16.
  if (kGateUp) {
    const int f = ncol[0];  // gate column == h column
    const float sg = wscale[(size_t)e * 2 * F + f];
    const float su = wscale[(size_t)e * 2 * F + F + f];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = rt * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        const bool valid = m0 + m < R;
        float hv = 0.0f;
        if (valid) {
          const int row = row0 + m0 + m;
          const float sxv = row_scale[m];
          const float g = (float)acc[rt][0][i] * sxv * sg;
          const float u = (float)acc[rt][1][i] * sxv * su;
          hv = g / (1.0f + expf(-g)) * u;
          static_cast<float *>(out_v)[(size_t)row * F + f] = hv;
          if (acc1_dbg) {
            acc1_dbg[(size_t)row * 2 * F + f] = acc[rt][0][i];
            acc1_dbg[(size_t)row * 2 * F + F + f] = acc[rt][1][i];
          }
        }
        float mx = __builtin_fabsf(hv);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o, 64));
        if (valid && (lane & 31) == 0) atomicMax(amax + row0 + m0 + m, __float_as_uint(mx));
      }
    }
  } else {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int n = ncol[ct];
      const float sd = wscale[(size_t)e * H + n];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = rt * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
          if (m0 + m < R) {
            const int row = row0 + m0 + m;
            static_cast<float *>(out_v)[(size_t)row * H + n] =
                (float)acc[rt][ct][i] * row_scale[m] * sd;
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm1_tiled(const int8_t *qx, const float *sx, const int32_t *sorted, int k,
                              const int32_t *counts, const int32_t *offsets,
                              const int32_t *mtile_off, int64_t A, const int8_t *w_gu,
                              const float *s_gu, int H, int F, int E, float *h, uint32_t *amax,
                              int32_t *acc1_dbg, hipStream_t st, Timing tm) {
  const int64_t mtiles = (A + BM - 1) / BM + E;
  const dim3 grid((unsigned)mtiles, (unsigned)(F / 128));
  return launch_kernel(gemm_tiled_kernel<true>, grid, dim3(256), st, tm, qx, sx, sorted, k, counts,
                       offsets, mtile_off, E, w_gu, s_gu, H, F, H, (void *)h, amax, acc1_dbg);
}

hipError_t launch_gemm2_tiled(const int8_t *qh, const float *sh, const int32_t *counts,
                              const int32_t *offsets, const int32_t *mtile_off, int64_t A,
                              const int8_t *w_d, const float *s_d, int H, int F, int E,
                              float *y, hipStream_t st, Timing tm) {
  const int64_t mtiles = (A + BM - 1) / BM + E;
  const dim3 grid((unsigned)mtiles, (unsigned)(H / 256));
  return launch_kernel(gemm_tiled_kernel<false>, grid, dim3(256), st, tm, qh, sh,
                       (const int32_t *)nullptr, 1, counts, offsets, mtile_off, E, w_d, s_d, F, F,
                       H, (void *)y, (uint32_t *)nullptr, (int32_t *)nullptr);
}

}  // namespace moe
