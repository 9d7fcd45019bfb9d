// router.hip -- the router projection in front of the top-k: logits = x . W_r^T.
//
// "超大规模模型推理的Day0适配实践" §四: the expert layer's gate is one of the
// small operators that belong inside the fused MoE operator, and the top-k it
// feeds must match exactly, tie-break included. "MiniMax-M3 W8A8 inference on
// K100AI" §6.1: the layers next to the routing stay in 16-bit floating point
// rather than INT8. So the projection takes the bf16 tokens and a bf16 router
// matrix and accumulates in fp32 on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16: products of bf16 are exact in fp32).
//
// The sum over the hidden dimension has a fixed order that depends on H
// only, so that a token's logits (and hence its experts) do not depend on
// the batch it arrives in: H is cut into parts of kRouterPart channels; in a
// part, wavefront w (of 4) runs the matrix-instruction chain over channels
// [part + 128 w, part + 128 w + 128), and the part's value is
// ((w0 + w1) + w2) + w3; the logit is the sum of the parts in order. The
// projection writes one fp32 plane per part ([parts][T][E]); the routing
// kernels add the planes in order as they read a token's logits, and
// router_sum_kernel does the same into a [T][E] array.
//
// Block = 4 wavefronts, 32 tokens x 64 experts of one part: lane l holds the
// 8 bf16 of row l%32 at channels 8*(l/32).. of each 16-channel step, for A
// (tokens) and for both 32-expert halves of B.
#include "layer_device.h"

namespace moe {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8bf as_bf16x8(v4i v) { return __builtin_bit_cast(v8bf, v); }

__global__ __launch_bounds__(256) void router_proj_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ wr,
                                                          int64_t T, int E, int H,
                                                          float *__restrict__ part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const int e0 = blockIdx.y * 64;
  const int s = blockIdx.z;
  const int r = lane & 31, kh = (lane >> 5) * 8;
  const int k_lo = s * kRouterPart + wave * 128;
  // Rows past T and experts past E repeat the last one; they are not stored.
  const int64_t tok = t0 + r < T ? t0 + r : T - 1;
  const int ea = e0 + r < E ? e0 + r : E - 1;
  const int eb = e0 + 32 + r < E ? e0 + 32 + r : E - 1;
  v16f acc0, acc1;
#pragma unroll
  for (int v = 0; v < 16; ++v) { acc0[v] = 0.0f; acc1[v] = 0.0f; }
  // H is a multiple of 256, so a wavefront's 128-channel run lies inside H
  // or entirely past it (then its sum is 0). All eight 16-channel steps are
  // loaded before the first matrix instruction.
  if (k_lo < H) {
    const uint16_t *pa = x + tok * H + k_lo + kh;
    const uint16_t *pb0 = wr + (int64_t)ea * H + k_lo + kh;
    const uint16_t *pb1 = wr + (int64_t)eb * H + k_lo + kh;
    v4i a[8], b0[8], b1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = *reinterpret_cast<const v4i *>(pa + 16 * i);
      b0[i] = *reinterpret_cast<const v4i *>(pb0 + 16 * i);
      b1[i] = *reinterpret_cast<const v4i *>(pb1 + 16 * i);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(b0[i]), acc0,
                                                     0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(b1[i]), acc1,
                                                     0, 0, 0);
    }
  }
  // ((w0 + w1) + w2) + w3, element by element.
  __shared__ float red[3][2][16][64];
  if (wave > 0) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      red[wave - 1][0][v][lane] = acc0[v];
      red[wave - 1][1][v][lane] = acc1[v];
    }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      acc0[v] += red[w][0][v][lane];
      acc1[v] += red[w][1][v][lane];
    }
  // Lane holds expert column r of each half and token rows
  // 8*(v/4) + 4*(lane/32) + v%4.
  float *plane = part + (int64_t)s * T * E;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t t = t0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (t < T) {
      if (e0 + r < E) plane[t * E + e0 + r] = acc0[v];
      if (e0 + 32 + r < E) plane[t * E + e0 + 32 + r] = acc1[v];
    }
  }
}

// logits[t][e] = sum of the part planes in order.
__global__ __launch_bounds__(256) void router_sum_kernel(const float *__restrict__ part,
                                                         int nparts, int64_t n,
                                                         float *__restrict__ logits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = part[i];
  for (int s = 1; s < nparts; ++s) v += part[(int64_t)s * n + i];
  logits[i] = v;
}

}  // namespace

int router_parts(int H) { return (H + kRouterPart - 1) / kRouterPart; }

hipError_t launch_router_proj(const uint16_t *x, const uint16_t *w_router, int64_t T, int E,
                              int H, float *part, hipStream_t st, Timing tm) {
  const dim3 grid((unsigned)((T + 31) / 32), (unsigned)((E + 63) / 64),
                  (unsigned)router_parts(H));
  return launch_kernel(router_proj_kernel, grid, dim3(256), st, tm, x, w_router, T, E, H, part);
}

hipError_t launch_router_sum(const float *part, int nparts, int64_t T, int E, float *logits,
                             hipStream_t st) {
  const int64_t n = T * E;
  return launch_kernel(router_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), st,
                       Timing{}, part, nparts, n, logits);
}

}  // namespace moe
