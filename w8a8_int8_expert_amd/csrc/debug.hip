// debug.hip -- the optional per-stage outputs of moe_w8a8_forward in the
// order the ABI defines them (dense permuted rows, row-major).
//
// Inside the layer every expert's group of permuted rows starts on a 16-row
// boundary and qh is fragment-tiled (the GEMM operand layout). Dense row i of
// expert e (offsets[e] <= i < offsets[e+1]) is padded row
// poffsets[e] + i - offsets[e]. These kernels run only when a caller asks
// for the stage outputs; they are not part of the layer's work.
#include "layer_device.h"

namespace moe {
namespace {

// One block per dense row: sorted, h, qh (untiled), sh and y of that row.
__global__ __launch_bounds__(256) void debug_rows_kernel(
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ poffsets, int E,
    const int32_t *__restrict__ sorted_p, const float *__restrict__ h_p,
    const int8_t *__restrict__ qh_t, const float *__restrict__ sh_p,
    const YRows y_p, int F, int H, int32_t *__restrict__ sorted,
    float *__restrict__ h, int8_t *__restrict__ qh, float *__restrict__ sh,
    float *__restrict__ y) {
  const int i = blockIdx.x;
  if (i >= offsets[E]) return;
  int lo = 0, hi = E;  // largest e with offsets[e] <= i
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= i) lo = mid; else hi = mid;
  }
  const size_t p = (size_t)(poffsets[lo] + i - offsets[lo]);
  const int tid = threadIdx.x;
  if (tid == 0) {
    if (sorted) sorted[i] = sorted_p[p];
    if (sh) sh[i] = sh_p[p];
  }
  for (int j = tid; j < F; j += 256) {
    if (h) h[(size_t)i * F + j] = h_p[p * F + j];
    if (qh) {
      const size_t at = frag_tile((int)(p >> 4), j >> 6, F) +
                        (size_t)(((((j & 63) >> 4) << 4) + (int)(p & 15)) << 4) + (j & 15);
      qh[(size_t)i * F + j] = qh_t[at];
    }
  }
  // y as the combine reads it (int16 rows: code times its group's scale)
  if (y)
    for (int j = tid; j < H; j += 256)
      y[(size_t)i * H + j] =
          y_p.f ? y_p.f[p * H + j]
                : (float)y_p.q[p * H + j] * y_p.s[p * (size_t)(H / kYGroup) + j / kYGroup];
}

// row_of in dense rows: padded row p of assignment a (expert ids[a]) maps
// to p - poffsets[e] + offsets[e]; -1 stays -1.
__global__ __launch_bounds__(256) void debug_row_of_kernel(const int32_t *__restrict__ row_of_p,
                                                           const int32_t *__restrict__ ids,
                                                           const int32_t *__restrict__ offsets,
                                                           const int32_t *__restrict__ poffsets,
                                                           int64_t A, int32_t *__restrict__ row_of) {
  const int64_t a = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (a >= A) return;
  const int32_t p = row_of_p[a];
  int32_t d = -1;
  if (p >= 0) {
    const int e = ids[a];
    d = p - poffsets[e] + offsets[e];
  }
  row_of[a] = d;
}

}  // namespace

hipError_t launch_debug_rows(const int32_t *offsets, const int32_t *poffsets, int E, int64_t A,
                             const int32_t *sorted_p, const float *h_p, const int8_t *qh_t,
                             const float *sh_p, YRows y_p, int F, int H, int32_t *sorted,
                             float *h, int8_t *qh, float *sh, float *y, hipStream_t st) {
  return launch_kernel(debug_rows_kernel, dim3((unsigned)A), dim3(256), st, Timing{}, offsets,
                       poffsets, E, sorted_p, h_p, qh_t, sh_p, y_p, F, H, sorted, h, qh, sh, y);
}

hipError_t launch_debug_row_of(const int32_t *row_of_p, const int32_t *ids, const int32_t *offsets,
                               const int32_t *poffsets, int64_t A, int32_t *row_of,
                               hipStream_t st) {
  return launch_kernel(debug_row_of_kernel, dim3((unsigned)((A + 255) / 256)), dim3(256), st,
                       Timing{}, row_of_p, ids, offsets, poffsets, A, row_of);
}

}  // namespace moe
