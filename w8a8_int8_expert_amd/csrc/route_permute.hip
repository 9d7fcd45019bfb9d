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
// Three launches:
//   route_hist  one block per 64 tokens: route (or copy pre-routed ids),
//               per-block expert histogram in LDS, clear the row max buffer;
//   scan        one block: per-expert exclusive scan over blocks, capacity,
//               expert offsets and the M-tile table of the tiled GEMMs;
//   scatter     one block per 64 tokens: stable ranks from wave ballots,
//               writes sorted[] and row_of[].
#include "moe_internal.h"

namespace moe {
namespace {

// (value, index) ordering of the router: higher logit first, then lower
// index. Comparisons are IEEE (so -0.0 ties +0.0). idx == INT32_MAX marks
// "no candidate"; a NaN never beats a candidate, so the winner is always a
// valid untaken expert.
__device__ __forceinline__ bool route_better(float av, int ai, float bv, int bi) {
  if (ai == INT32_MAX) return false;
  if (bi == INT32_MAX) return true;
  return av > bv || (av == bv && ai < bi);
}

__global__ __launch_bounds__(256) void route_hist_kernel(
    const float *__restrict__ logits, const int32_t *__restrict__ ids_in,
    const float *__restrict__ w_in, int64_t T, int E, int k, int32_t *__restrict__ ids,
    float *__restrict__ wts, int32_t *__restrict__ blk_hist, uint32_t *__restrict__ amax) {
  __shared__ int32_t hist[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  // Clear the per-row max of this block's share of permuted rows (rows are
  // < T*k; block b owns [b*64*k, (b+1)*64*k)).
  {
    const int64_t A = T * (int64_t)k;
    const int64_t r0 = (int64_t)blockIdx.x * kRouteTokens * k;
    const int64_t r1 = r0 + (int64_t)kRouteTokens * k < A ? r0 + (int64_t)kRouteTokens * k : A;
    for (int64_t r = r0 + tid; r < r1; r += 256) amax[r] = 0u;
  }
  __syncthreads();
  const int64_t t0 = (int64_t)blockIdx.x * kRouteTokens;
  for (int tt = wave; tt < kRouteTokens; tt += 4) {
    const int64_t t = t0 + tt;
    if (t >= T) break;
    if (logits == nullptr) {
      if (lane < k) {
        const int32_t e = ids_in[t * k + lane];
        ids[t * k + lane] = e;
        wts[t * k + lane] = w_in[t * k + lane];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
      }
      continue;
    }
    // Lane holds experts lane, lane+64, ...; `taken` marks chosen ones.
    float v[kMaxExperts / 64];
    uint32_t taken = 0;
    const float *row = logits + t * E;
#pragma unroll
    for (int i = 0; i < kMaxExperts / 64; ++i) {
      const int e = lane + 64 * i;
      if (e < E) v[i] = row[e];
      else { v[i] = 0.0f; taken |= 1u << i; }
    }
    float my_logit = 0.0f;
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
      float bv = 0.0f;
      int bi = INT32_MAX;
#pragma unroll
      for (int i = 0; i < kMaxExperts / 64; ++i) {
        if (taken & (1u << i)) continue;
        if (route_better(v[i], lane + 64 * i, bv, bi)) { bv = v[i]; bi = lane + 64 * i; }
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (route_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == j) { my_logit = bv; my_id = bi; }
    }
    // Renormalised softmax over the chosen k: exp(l_j - l_0) / sum.
    const float m = __shfl(my_logit, 0, 64);
    const float ex = lane < k ? expf(my_logit - m) : 0.0f;
    const float den = wave_sum(ex);
    if (lane < k) {
      ids[t * k + lane] = my_id;
      wts[t * k + lane] = ex / den;
      atomicAdd(&hist[my_id], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) blk_hist[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Inclusive wave scan of ints (64 lanes).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// One block of 1024 threads. Wave w scans the block histograms of experts
// w, w+16, ...: blk_hist[b][e] becomes the number of assignments to e in
// blocks before b. Then capacity, offsets and the M-tile table.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t *__restrict__ blk_hist, int64_t nblk,
                                                    int E, int64_t capacity,
                                                    int32_t *__restrict__ counts,
                                                    int32_t *__restrict__ offsets,
                                                    int32_t *__restrict__ mtile_off) {
  __shared__ int32_t total[kMaxExperts];
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t per_lane = (nblk + 63) / 64;
  for (int e = wave; e < E; e += 16) {
    const int64_t b0 = lane * per_lane;
    const int64_t b1 = b0 + per_lane < nblk ? b0 + per_lane : nblk;
    int s = 0;
    for (int64_t b = b0; b < b1; ++b) s += blk_hist[b * E + e];
    const int incl = wave_incl_scan(s);
    int run = incl - s;  // exclusive prefix of this lane's first block
    for (int64_t b = b0; b < b1; ++b) {
      const int c = blk_hist[b * E + e];
      blk_hist[b * E + e] = run;
      run += c;
    }
    if (lane == 63) total[e] = incl;
  }
  __syncthreads();
  // Kept counts and their exclusive scans (E <= 1024 = one per thread).
  int kept = 0, tiles = 0;
  if (tid < E) {
    kept = total[tid];
    if (capacity > 0 && (int64_t)kept > capacity) kept = (int)capacity;
    tiles = (kept + kTiledBM - 1) / kTiledBM;
    counts[tid] = kept;
  }
  // Block-wide exclusive scans of the kept counts (-> offsets) and of the
  // M tiles per expert (-> mtile_off), one after the other.
  for (int pass = 0; pass < 2; ++pass) {
    const int v = pass == 0 ? kept : tiles;
    const int incl = wave_incl_scan(v);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    int32_t *dst = pass == 0 ? offsets : mtile_off;
    if (tid < E) dst[tid] = base + incl - v;
    if (tid == E - 1) dst[E] = base + incl;
    __syncthreads();
  }
}

// Stable scatter. Assignments of this block are processed in rounds of 256
// (4 waves x 64 lanes, wave order = assignment order). A lane's rank among
// equal experts of its wave comes from ballots over the id bits; earlier
// waves of the round and earlier rounds are added through LDS counters.
__global__ __launch_bounds__(256) void scatter_kernel(
    const int32_t *__restrict__ ids, const int32_t *__restrict__ blk_base,
    const int32_t *__restrict__ offsets, int64_t T, int E, int k, int64_t capacity,
    int32_t *__restrict__ sorted, int32_t *__restrict__ row_of) {
  __shared__ int32_t running[kMaxExperts];
  __shared__ int32_t wcnt[4][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 256) {
    running[e] = blk_base[(int64_t)blockIdx.x * E + e];
    wcnt[0][e] = wcnt[1][e] = wcnt[2][e] = wcnt[3][e] = 0;
  }
  __syncthreads();
  const int64_t A = T * (int64_t)k;
  const int64_t a0 = (int64_t)blockIdx.x * kRouteTokens * k;
  const int64_t a1 = a0 + (int64_t)kRouteTokens * k < A ? a0 + (int64_t)kRouteTokens * k : A;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t base = a0; base < a1; base += 256) {
    const int64_t a = base + tid;
    int e = -1;
    if (a < a1) {
      e = ids[a];
      if (e < 0 || e >= E) e = -1;
    }
    const bool valid = e >= 0;
    uint64_t mask = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t bal = __ballot(bit);
      mask &= bit ? bal : ~bal;
    }
    const int rank = __popcll(mask & lt_mask);
    const int cnt = __popcll(mask);
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

}  // namespace

hipError_t launch_route_hist(const float *logits, const int32_t *ids_in, const float *w_in,
                             int64_t T, int E, int k, int32_t *ids, float *wts,
                             int32_t *blk_hist, uint32_t *amax, hipStream_t st) {
  const int64_t nblk = (T + kRouteTokens - 1) / kRouteTokens;
  route_hist_kernel<<<dim3((unsigned)nblk), dim3(256), 0, st>>>(logits, ids_in, w_in, T, E, k,
                                                                 ids, wts, blk_hist, amax);
  return hipGetLastError();
}

hipError_t launch_scan(int32_t *blk_hist, int64_t nblk, int E, int64_t capacity, int32_t *counts,
                       int32_t *offsets, int32_t *mtile_off, hipStream_t st) {
  scan_kernel<<<dim3(1), dim3(1024), 0, st>>>(blk_hist, nblk, E, capacity, counts, offsets,
                                               mtile_off);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t *ids, const int32_t *blk_hist, const int32_t *offsets,
                          int64_t T, int E, int k, int64_t capacity, int32_t *sorted,
                          int32_t *row_of, hipStream_t st) {
  const int64_t nblk = (T + kRouteTokens - 1) / kRouteTokens;
  scatter_kernel<<<dim3((unsigned)nblk), dim3(256), 0, st>>>(ids, blk_hist, offsets, T, E, k,
                                                              capacity, sorted, row_of);
  return hipGetLastError();
}

}  // namespace moe
