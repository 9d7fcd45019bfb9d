// pack.hip -- the fragment-tiled layout of quantised weights from row-major
// codes ("MiniMax-M3 W8A8 inference on K100AI", mhpq.cn/news/1068415,
// §3.2-§3.3: weights quantised offline by one tool are then built into the
// engine's own layout). The layout is the one include/moe_w8a8.h defines:
// 1 KB tiles of 16 rows x 64 k, tile (n/16, k/64) at ((n/16)*(K/64) + k/64)
// KB, element (n, k) at byte (((k%64)/16)*16 + n%16)*16 + k%16 of its tile.
// Every 16-byte chunk of a tile is 16 consecutive codes of one source row, so
// one thread copies one chunk: the stores of a wavefront are 1 KB contiguous,
// its loads four 64-byte pieces of 16 rows.
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void pack_kernel(const int8_t *__restrict__ src,
                                                   int8_t *__restrict__ dst, int64_t chunks,
                                                   int N, int K) {
  const int64_t per_matrix = (int64_t)N * K / 16;  // 16-byte chunks per matrix
  const int kt_per_row = K / 64;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = i / per_matrix;
    const int64_t j = i - c * per_matrix;
    const int64_t tile = j >> 6;  // 64 chunks per 1 KB tile
    const int q = (int)(j & 63);
    const int64_t n_tile = tile / kt_per_row;
    const int k_tile = (int)(tile - n_tile * kt_per_row);
    const int64_t n = n_tile * 16 + (q & 15);
    const int64_t k = (int64_t)k_tile * 64 + (q >> 4) * 16;
    const v4i v = *reinterpret_cast<const v4i *>(src + c * (int64_t)N * K + n * K + k);
    *reinterpret_cast<v4i *>(dst + i * 16) = v;
  }
}

}  // namespace

hipError_t launch_pack(const int8_t *src, int8_t *dst, int64_t count, int N, int K,
                       hipStream_t st) {
  const int64_t chunks = count * (int64_t)N * K / 16;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return launch_kernel(pack_kernel, dim3((unsigned)blocks), dim3(256), st, Timing{}, src, dst,
                       chunks, N, K);
}

}  // namespace moe
