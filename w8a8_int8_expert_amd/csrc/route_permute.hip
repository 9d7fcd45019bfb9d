// route_permute.hip -- top-k routing and the expert grouping of assignments.
//
// Routing follows "超大规模模型推理的Day0适配实践" §四 (the fused MoE operator:
// gate, sort, un-sort, weighted sum; its top-k must reproduce the reference
// exactly, tie-break included): experts ordered by (logit descending, index
// ascending), the first k taken, softmax weights renormalised over them.
// Grouping ("sort") is a histogram + prefix scan + stable scatter, so the
// order inside an expert group is (token, slot) and the capacity rule of the
// same page (§二.2, capacity factor; overflow dropped) keeps the first C.
//
// Two ways through, chosen by the number of assignments A = T*k:
//  small A (a decode step): ONE launch, prologue_small_kernel. Block 0 routes
//      every token (one wavefront per token, the next token's logits loaded
//      before the current one is ranked), histograms in LDS, scans the
//      counts in one packed block scan, and scatters stably with four
//      wavefronts' ballots; blocks 1.. quantise the activations (one
//      wavefront per token) at the same time.
//  large A (prefill): route_hist (one block per tpb = route_tokens(T)
//      tokens, 16 to 64: route, per-block LDS histogram) -> scan (one block:
//      per-expert scan over blocks, capacity, offsets, M-tile table) ->
//      scatter (one block per tpb tokens: stable ranks from wave ballots);
//      activation quantisation is its own launch (quant.hip).
// Inside the layer every expert's group of permuted rows starts on a 16-row
// boundary ("padded" rows: the activation operands of the grouped GEMMs are
// stored as 16-row x 64-k tiles, and no tile may hold two experts' rows).
// Both paths write the dense offsets (the grouping as the order defines it),
// the padded offsets, sorted[] and row_of[] in padded rows (-1 marks padding
// and dropped assignments), and clear the per-row max buffer that GEMM1
// fills later in the call.
#include "layer_device.h"

namespace moe {
namespace {

// Stable rank of each lane's expert among the lanes before it with the same
// expert (ballots over the id bits); -1 ids never match a valid one.
__device__ __forceinline__ void ballot_rank(int e, bool valid, int nbits, int *rank, int *cnt) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t mask = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t bal = __ballot(bit);
    mask &= bit ? bal : ~bal;
  }
  *rank = __popcll(mask & lt_mask);
  *cnt = __popcll(mask);
}

__device__ __forceinline__ int id_bits(int E) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

// Fill n int32 words starting at p with v, with the threads of this block.
__device__ __forceinline__ void block_fill(uint32_t *p, int64_t n, uint32_t v) {
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) p[i] = v;
}

// Block-wide exclusive scan of one int per thread (blockDim.x == 1024);
// returns the exclusive prefix, *total gets the sum. Uses wsum[16].
__device__ __forceinline__ int block_excl_scan(int v, int *wsum, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) base += wsum[w];
    all += wsum[w];
  }
  __syncthreads();
  *total = all;
  return base + incl - v;
}

// Kept counts per expert from the totals: capacity, dense offsets, 16-row
// aligned (padded) offsets, counts and the M-tile table of the tiled GEMMs.
// One thread per expert (E <= 1024, 1024 threads). Returns this thread's
// padded offset (0 past E).
__device__ __forceinline__ int finish_counts(int total, int E, int64_t capacity,
                                             int32_t *__restrict__ counts,
                                             int32_t *__restrict__ offsets,
                                             int32_t *__restrict__ poffsets,
                                             int32_t *__restrict__ mtile_off, int *wsum) {
  const int tid = threadIdx.x;
  int kept = 0, tiles = 0, padded = 0;
  if (tid < E) {
    kept = total;
    if (capacity > 0 && (int64_t)kept > capacity) kept = (int)capacity;
    tiles = (kept + kTiledBM - 1) / kTiledBM;
    padded = (kept + 15) & ~15;
    counts[tid] = kept;
  }
  int all;
  const int off = block_excl_scan(kept, wsum, &all);
  if (tid < E) offsets[tid] = off;
  if (tid == 0) offsets[E] = all;
  const int poff = block_excl_scan(padded, wsum, &all);
  if (tid < E) poffsets[tid] = poff;
  if (tid == 0) poffsets[E] = all;
  const int toff = block_excl_scan(tiles, wsum, &all);
  if (tid < E) mtile_off[tid] = toff;
  if (tid == 0) mtile_off[E] = all;
  return poff;
}

// finish_counts for at most kSmallA assignments, with one block scan: kept
// count, padded count and M tiles of an expert packed into 21-bit fields of
// one 64-bit value (each field's total stays below 2^21 for A <= kSmallA and
// E <= kMaxExperts, so no field carries into the next).
__device__ __forceinline__ int finish_counts_small(int total, int E, int64_t capacity,
                                                   int32_t *__restrict__ counts,
                                                   int32_t *__restrict__ offsets,
                                                   int32_t *__restrict__ poffsets,
                                                   int32_t *__restrict__ mtile_off,
                                                   uint64_t *wsum) {
  static_assert(kSmallA + 15 * kMaxExperts < (1 << 21) && kSmallA / kTiledBM + kMaxExperts < (1 << 21),
                "packed fields");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t v = 0;
  if (tid < E) {
    int kept = total;
    if (capacity > 0 && (int64_t)kept > capacity) kept = (int)capacity;
    counts[tid] = kept;
    v = (uint64_t)kept | ((uint64_t)((kept + 15) & ~15) << 21) |
        ((uint64_t)((kept + kTiledBM - 1) / kTiledBM) << 42);
  }
  const uint64_t incl = wave_incl_scan_u64(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint64_t base = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) base += wsum[w];
    all += wsum[w];
  }
  const uint64_t ex = base + incl - v;
  constexpr uint64_t kField = (1u << 21) - 1;
  const int poff = (int)((ex >> 21) & kField);
  if (tid < E) {
    offsets[tid] = (int)(ex & kField);
    poffsets[tid] = poff;
    mtile_off[tid] = (int)(ex >> 42);
  }
  if (tid == 0) {
    offsets[E] = (int)(all & kField);
    poffsets[E] = (int)((all >> 21) & kField);
    mtile_off[E] = (int)(all >> 42);
  }
  return poff;
}

// ------------------------------------------------------------- small A path
constexpr int kSmallQuantTokens = 4;  // tokens quantised per block (blocks 1..)

template <int NV>
__global__ __launch_bounds__(1024) void prologue_small_kernel(
    const LogitPlanes logits, const int32_t *__restrict__ ids_in,
    const float *__restrict__ w_in, int T, int E, int k, int64_t capacity,
    int32_t *__restrict__ ids, float *__restrict__ wts, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ poffsets,
    int32_t *__restrict__ mtile_off, int32_t *__restrict__ sorted, int32_t *__restrict__ row_of,
    int P, const uint16_t *__restrict__ x, const float *__restrict__ inv_s, int H,
    int8_t *__restrict__ qx, float *__restrict__ sx, uint32_t *__restrict__ amax, ActClip ac,
    bool fp8) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x > 0) {
    // Four tokens per block: the quantisation is spread over many compute
    // units instead of stacking 16 wavefronts' arithmetic on one.
    const int64_t t = (int64_t)(blockIdx.x - 1) * kSmallQuantTokens + wave;
    if (wave < kSmallQuantTokens && t < T)
      quant_token_row<16>(x + t * H, inv_s, H, qx + t * H, sx + t, ac, fp8);
    return;
  }
  __shared__ uint64_t wave_keys[16][64];
  __shared__ int32_t hist[kMaxExperts];
  __shared__ int32_t run[kMaxExperts];
  __shared__ int32_t lds_ids[kSmallA];
  __shared__ int32_t lds_off[kMaxExperts];
  __shared__ int32_t wcnt[4][kMaxExperts];
  __shared__ uint64_t wsum[16];
  const int A = T * k;
  for (int e = tid; e < E; e += 1024) {
    hist[e] = 0;
    run[e] = 0;
    wcnt[0][e] = wcnt[1][e] = wcnt[2][e] = wcnt[3][e] = 0;
  }
  block_fill(amax, P, 0u);
  block_fill(reinterpret_cast<uint32_t *>(sorted), P, 0xFFFFFFFFu);
  __syncthreads();
  // Up to 64 experts the next token's logits are loaded before this one is
  // routed, so their latency overlaps the routing.
  float cur = 0.0f;
  if (NV == 1 && logits.p && wave < T && lane < E)
    cur = logit_of(logits, logits.p + (int64_t)wave * E, lane);
  for (int t = wave; t < T; t += 16) {
    int e;
    float w;
    if (NV == 1 && logits.p) {
      float nxt = 0.0f;
      if (t + 16 < T && lane < E) nxt = logit_of(logits, logits.p + (int64_t)(t + 16) * E, lane);
      e = route_logit_wave(cur, E, k, &w, wave_keys[wave]);
      cur = nxt;
    } else if (logits.p) {
      e = route_token_wave<NV>(logits, t, E, k, &w, wave_keys[wave]);
    } else {
      e = lane < k ? ids_in[t * k + lane] : -1;
      w = lane < k ? w_in[t * k + lane] : 0.0f;
    }
    if (lane < k) {
      ids[t * k + lane] = e;
      wts[t * k + lane] = w;
      lds_ids[t * k + lane] = e;
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  const int off = finish_counts_small(tid < E ? hist[tid] : 0, E, capacity, counts, offsets,
                                      poffsets, mtile_off, wsum);
  if (tid < E) lds_off[tid] = off;
  __syncthreads();
  // Stable scatter by waves 0..3, 256 assignments per round (wave order =
  // assignment order): a lane's rank among equal experts of its wave from
  // ballots, plus earlier waves of the round and earlier rounds through LDS
  // counters. Every wave takes part in the barriers.
  const int nbits = id_bits(E);
  for (int base = 0; base < A; base += 256) {
    const int a = base + 64 * wave + lane;
    int e = wave < 4 && a < A ? lds_ids[a] : -1;
    const bool valid = e >= 0 && e < E;
    if (!valid) e = -1;
    int rank = 0, cnt = 0;
    if (wave < 4) ballot_rank(e, valid, nbits, &rank, &cnt);
    const bool leader = valid && rank == cnt - 1;
    if (leader) wcnt[wave][e] = cnt;
    __syncthreads();
    if (wave < 4 && a < A) {
      int32_t row = -1;
      if (valid) {
        int r = run[e] + rank;
        for (int w = 0; w < wave; ++w) r += wcnt[w][e];
        if (capacity <= 0 || (int64_t)r < capacity) {
          row = lds_off[e] + r;
          sorted[row] = a;
        }
      }
      row_of[a] = row;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&run[e], cnt);
      wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------- large A path
template <int NV>
__global__ __launch_bounds__(1024) void route_hist_kernel(
    const LogitPlanes logits, const int32_t *__restrict__ ids_in,
    const float *__restrict__ w_in, int64_t T, int E, int k, int32_t *__restrict__ ids,
    float *__restrict__ wts, int32_t *__restrict__ blk_hist, uint32_t *__restrict__ amax,
    int32_t *__restrict__ sorted, int64_t P, int tpb) {
  __shared__ uint64_t wave_keys[16][64];
  __shared__ int32_t hist[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 1024) hist[e] = 0;
  // This block's share of the padded rows: [b*tpb*k, (b+1)*tpb*k), and the
  // last block also takes the rows past T*k.
  {
    const int64_t r0 = (int64_t)blockIdx.x * tpb * k;
    int64_t r1 = r0 + (int64_t)tpb * k;
    if (blockIdx.x == gridDim.x - 1 || r1 > P) r1 = P;
    for (int64_t r = r0 + tid; r < r1; r += 1024) {
      amax[r] = 0u;
      sorted[r] = -1;
    }
  }
  __syncthreads();
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  for (int tt = wave; tt < tpb; tt += 16) {
    const int64_t t = t0 + tt;
    if (t >= T) break;
    int e;
    float w;
    if (logits.p) {
      e = route_token_wave<NV>(logits, t, E, k, &w, wave_keys[wave]);
    } else {
      e = lane < k ? ids_in[t * k + lane] : -1;
      w = lane < k ? w_in[t * k + lane] : 0.0f;
    }
    if (lane < k) {
      ids[t * k + lane] = e;
      wts[t * k + lane] = w;
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) blk_hist[(int64_t)e * gridDim.x + blockIdx.x] = hist[e];
}

// One block of 1024 threads. Wave w scans the block histograms of experts
// w, w+16, ... (stored expert-major, blk_hist[e][b], so a lane reads a
// contiguous run of blocks): blk_hist[e][b] becomes the number of
// assignments to e in blocks before b. Then capacity, offsets and the M-tile
// table.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t *__restrict__ blk_hist, int64_t nblk,
                                                    int E, int64_t capacity,
                                                    int32_t *__restrict__ counts,
                                                    int32_t *__restrict__ offsets,
                                                    int32_t *__restrict__ poffsets,
                                                    int32_t *__restrict__ mtile_off) {
  __shared__ int32_t total[kMaxExperts];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t per_lane = (nblk + 63) / 64;
  const int64_t b0 = lane * per_lane;
  const int64_t b1 = b0 + per_lane < nblk ? b0 + per_lane : nblk;
  if (per_lane <= 4) {
    // At most 256 blocks: four experts per wavefront at a time, every load
    // of the four issued before the scans, so their latencies overlap.
    constexpr int G = 4;
    for (int e0 = wave; e0 < E; e0 += 16 * G) {
      int c[G][4], s[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int e = e0 + 16 * g;
        const int32_t *row = blk_hist + (int64_t)(e < E ? e : 0) * nblk;
#pragma unroll
        for (int j = 0; j < 4; ++j) c[g][j] = (e < E && b0 + j < b1) ? row[b0 + j] : 0;
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int e = e0 + 16 * g;
        s[g] = c[g][0] + c[g][1] + c[g][2] + c[g][3];
        const int incl = wave_incl_scan(s[g]);
        if (e < E) {
          int32_t *row = blk_hist + (int64_t)e * nblk;
          int r = incl - s[g];  // exclusive prefix of this lane's first block
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (b0 + j < b1) {
              row[b0 + j] = r;
              r += c[g][j];
            }
          if (lane == 63) total[e] = incl;
        }
      }
    }
  } else {
    for (int e = wave; e < E; e += 16) {
      int32_t *row = blk_hist + (int64_t)e * nblk;
      int s = 0;
#pragma unroll 8
      for (int64_t b = b0; b < b1; ++b) s += row[b];
      const int incl = wave_incl_scan(s);
      int r = incl - s;  // exclusive prefix of this lane's first block
      for (int64_t b = b0; b < b1; ++b) {
        const int c = row[b];
        row[b] = r;
        r += c;
      }
      if (lane == 63) total[e] = incl;
    }
  }
  __syncthreads();
  finish_counts(tid < E ? total[tid] : 0, E, capacity, counts, offsets, poffsets, mtile_off,
                wsum);
}

// Stable scatter into padded rows (`offsets` are the padded offsets here).
// Assignments of this block are processed in rounds of 256
// (4 waves x 64 lanes, wave order = assignment order). A lane's rank among
// equal experts of its wave comes from ballots over the id bits; earlier
// waves of the round and earlier rounds are added through LDS counters.
// Blocks past the nblk routing blocks build the tiled GEMMs' tile orders
// (8 per GEMM whose region is given), which need only the M-tile table.
__global__ __launch_bounds__(256) void scatter_kernel(
    const int32_t *__restrict__ ids, const int32_t *__restrict__ blk_base,
    const int32_t *__restrict__ offsets, int64_t T, int E, int k, int64_t capacity,
    int32_t *__restrict__ sorted, int32_t *__restrict__ row_of, int tpb, int nblk,
    const TileOrderArgs to) {
  if ((int)blockIdx.x >= nblk) {
    const int b = (int)blockIdx.x - nblk;
    const int g = to.order[0] ? b >> 3 : 1;  // the blocks of GEMM 1's order come first
    tile_order_block(to, b & 7, g);
    return;
  }
  __shared__ int32_t running[kMaxExperts];
  __shared__ int32_t wcnt[4][kMaxExperts];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int e = tid; e < E; e += 256) {
    running[e] = blk_base[(int64_t)e * nblk + blockIdx.x];
    wcnt[0][e] = wcnt[1][e] = wcnt[2][e] = wcnt[3][e] = 0;
  }
  __syncthreads();
  const int64_t A = T * (int64_t)k;
  const int64_t a0 = (int64_t)blockIdx.x * tpb * k;
  const int64_t a1 = a0 + (int64_t)tpb * k < A ? a0 + (int64_t)tpb * k : A;
  const int nbits = id_bits(E);
  for (int64_t base = a0; base < a1; base += 256) {
    const int64_t a = base + tid;
    int e = -1;
    if (a < a1) {
      e = ids[a];
      if (e < 0 || e >= E) e = -1;
    }
    const bool valid = e >= 0;
    int rank, cnt;
    ballot_rank(e, valid, nbits, &rank, &cnt);
    const bool leader = valid && (rank == cnt - 1);
    if (leader) wcnt[wave][e] = cnt;
    __syncthreads();
    if (a < a1) {
      int32_t row = -1;
      if (valid) {
        int r = running[e] + rank;
        for (int w = 0; w < wave; ++w) r += wcnt[w][e];
        if (capacity <= 0 || (int64_t)r < capacity) {
          row = offsets[e] + r;
          sorted[row] = (int32_t)a;
        }
      }
      row_of[a] = row;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&running[e], cnt);
      wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

// Experts held per lane by the router: the smallest of 1, 2, 4, 8, 16 with
// 64 * NV >= E.
int route_nv(int E) {
  int nv = 1;
  while (64 * nv < E) nv *= 2;
  return nv;
}

}  // namespace

hipError_t launch_prologue_small(LogitPlanes logits, const int32_t *ids_in, const float *w_in,
                                 int T, int E, int k, int64_t capacity, int32_t *ids, float *wts,
                                 int32_t *counts, int32_t *offsets, int32_t *poffsets,
                                 int32_t *mtile_off, int32_t *sorted, int32_t *row_of, int P,
                                 const uint16_t *x, const float *inv_s, int H, int8_t *qx,
                                 float *sx, uint32_t *amax, ActClip ac, bool fp8,
                                 hipStream_t st, Timing tm) {
  const dim3 grid(1 + (unsigned)((T + kSmallQuantTokens - 1) / kSmallQuantTokens)), block(1024);
#define MOE_PROLOGUE(NV)                                                                     \
  return launch_kernel(prologue_small_kernel<NV>, grid, block, st, tm, logits, ids_in, w_in, T, \
                       E, k, capacity, ids, wts, counts, offsets, poffsets, mtile_off, sorted,  \
                       row_of, P, x, inv_s, H, qx, sx, amax, ac, fp8)
  switch (route_nv(E)) {
    case 1: MOE_PROLOGUE(1);
    case 2: MOE_PROLOGUE(2);
    case 4: MOE_PROLOGUE(4);
    case 8: MOE_PROLOGUE(8);
    default: MOE_PROLOGUE(16);
  }
#undef MOE_PROLOGUE
}

hipError_t launch_route_hist(LogitPlanes logits, const int32_t *ids_in, const float *w_in,
                             int64_t T, int E, int k, int32_t *ids, float *wts,
                             int32_t *blk_hist, uint32_t *amax, int32_t *sorted, int64_t P,
                             hipStream_t st, Timing tm) {
  const int tpb = route_tokens(T);
  const dim3 grid((unsigned)((T + tpb - 1) / tpb)), block(1024);
#define MOE_ROUTE(NV)                                                                        \
  return launch_kernel(route_hist_kernel<NV>, grid, block, st, tm, logits, ids_in, w_in, T, E, \
                       k, ids, wts, blk_hist, amax, sorted, P, tpb)
  switch (route_nv(E)) {
    case 1: MOE_ROUTE(1);
    case 2: MOE_ROUTE(2);
    case 4: MOE_ROUTE(4);
    case 8: MOE_ROUTE(8);
    default: MOE_ROUTE(16);
  }
#undef MOE_ROUTE
}

hipError_t launch_scan(int32_t *blk_hist, int64_t nblk, int E, int64_t capacity, int32_t *counts,
                       int32_t *offsets, int32_t *poffsets, int32_t *mtile_off, hipStream_t st,
                       Timing tm) {
  return launch_kernel(scan_kernel, dim3(1), dim3(1024), st, tm, blk_hist, nblk, E, capacity,
                       counts, offsets, poffsets, mtile_off);
}

hipError_t launch_scatter(const int32_t *ids, const int32_t *blk_hist, const int32_t *offsets,
                          int64_t T, int E, int k, int64_t capacity, int32_t *sorted,
                          int32_t *row_of, const TileOrderArgs &to, hipStream_t st, Timing tm) {
  const int tpb = route_tokens(T);
  const int64_t nblk = (T + tpb - 1) / tpb;
  const int extra = 8 * ((to.order[0] ? 1 : 0) + (to.order[1] ? 1 : 0));
  return launch_kernel(scatter_kernel, dim3((unsigned)(nblk + extra)), dim3(256), st, tm, ids,
                       blk_hist, offsets, T, E, k, capacity, sorted, row_of, tpb, (int)nblk, to);
}

}  // namespace moe
