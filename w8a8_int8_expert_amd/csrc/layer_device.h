// layer_device.h -- device building blocks of the layer shared by more than
// one kernel: the per-token router, the per-token INT8 quantiser and the
// gate-weighted combine of one token. Included by the HIP sources only.
#pragma once

#include "moe_internal.h"

namespace moe {

// ------------------------------------------------------------------ routing
// "超大规模模型推理的Day0适配实践" §四: the fused MoE operator's top-k must equal
// the reference exactly, tie-break included; ties go to the lower expert
// index. An expert is ranked by a 64-bit key: the upper half orders the
// logit (IEEE order, with -0.0 and +0.0 equal because the value is
// canonicalised by adding +0.0), the lower half is ~index so that the lower
// index wins a tie. A NaN logit gets the lowest order and is only chosen
// when nothing else is left; every valid expert's key is > 0, so 0 marks
// "taken" or "no expert".
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t o = 0u;
  if (v == v) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ int key_expert(uint64_t key) {
  return (int)(0xFFFFFFFFu - (uint32_t)key);
}
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Renormalised softmax over the chosen k, from slot j's key on lane j:
// exp(l_j - l_0) / sum over the k slots, summed in slot order.
__device__ __forceinline__ float topk_weight(uint64_t mine, int k) {
  const int lane = threadIdx.x & 63;
  const float l = key_logit(mine);
  const float m = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(l), 0));
  const float ex = lane < k ? expf(l - m) : 0.0f;
  float den = 0.0f;
  for (int j = 0; j < k; ++j)
    den += __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(ex), j));
  return ex / den;
}

// One wavefront routes token t: experts lane + 64*i (i < NV) are held by
// the lane. Up to 64 experts (NV = 1): the wavefront's keys go through its
// 64-entry LDS slot `keys`, every lane counts the keys above its own (keys
// are distinct), which is its expert's rank, and one permute moves the key of
// rank j to lane j. More experts: k rounds of a wave-wide key maximum pick
// the top k in order.
// Lane j < k returns slot j's expert and weight; other lanes return -1.
__device__ __forceinline__ float logit_of(const LogitPlanes &lp, const float *row, int e) {
  float v = row[e];
  for (int s = 1; s < lp.nparts; ++s) v += row[(int64_t)s * lp.stride + e];
  return v;
}

// Up to 64 experts, from the logit of expert `lane` already in hand (lanes
// past E ignore theirs).
__device__ __forceinline__ int route_logit_wave(float v, int E, int k, float *w_out,
                                                uint64_t *keys) {
  const int lane = threadIdx.x & 63;
  {
    const uint64_t key = lane < E ? route_key(v, lane) : 0ull;
    keys[lane] = key;
    // A wavefront's LDS accesses complete in issue order; keep the compiler
    // from moving the reads above the write.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int rank = 0;
#pragma unroll
    for (int j = 0; j < 64; j += 2) {
      const ulonglong2 kj = *reinterpret_cast<const ulonglong2 *>(keys + j);
      rank += (kj.x > key ? 1 : 0) + (kj.y > key ? 1 : 0);
    }
    __builtin_amdgcn_wave_barrier();
    // Lanes past E hold key 0 and share rank E >= k; their pushes land on
    // lanes that return -1.
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_permute(rank * 4, (int)(uint32_t)(key >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_permute(rank * 4, (int)(uint32_t)key);
    const uint64_t mine = ((uint64_t)hi << 32) | lo;
    *w_out = topk_weight(mine, k);
    return lane < k ? key_expert(mine) : -1;
  }
}

template <int NV>
__device__ __forceinline__ int route_token_wave(const LogitPlanes &lp, int64_t t, int E, int k,
                                                float *w_out, uint64_t *keys) {
  const int lane = threadIdx.x & 63;
  const float *row = lp.p + t * E;
  if (NV == 1) return route_logit_wave(lane < E ? logit_of(lp, row, lane) : 0.0f, E, k, w_out, keys);
  uint64_t key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? route_key(logit_of(lp, row, e), e) : 0ull;
  }
  uint64_t mine = 0ull;
  for (int j = 0; j < k; ++j) {
    uint64_t b = key[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) b = key[i] > b ? key[i] : b;
    b = wave_max_u64(b);
    const int e = key_expert(b);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i == e) key[i] = 0ull;
    if (lane == j) mine = b;
  }
  *w_out = topk_weight(mine, k);
  return lane < k ? key_expert(mine) : -1;
}

// ------------------------------------------------------------ quantisation
// Insert the bits of a non-negative float (which order as unsigned integers)
// into a lane's list of its kMaxSatM largest, kept in descending order.
__device__ __forceinline__ void top_insert(uint32_t (&l)[kMaxSatM], uint32_t v) {
#pragma unroll
  for (int s = kMaxSatM - 1; s > 0; --s) l[s] = v > l[s - 1] ? l[s - 1] : (v > l[s] ? v : l[s]);
  l[0] = v > l[0] ? v : l[0];
}

// m-th largest (m <= kMaxSatM) of the values the wavefront holds, given each
// lane's list of its kMaxSatM largest: the global m largest are all in the
// lists, so counting list entries >= a candidate decides every bit of the
// answer exactly. top = bits of the overall maximum.
__device__ __forceinline__ uint32_t wave_mth_largest(const uint32_t (&l)[kMaxSatM], int m,
                                                     uint32_t top) {
  uint32_t ans = 0u;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cand = ans | (1u << bit);
    if (cand > top) continue;  // nothing is >= cand
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < kMaxSatM; ++s) cnt += l[s] >= cand ? 1 : 0;
    cnt = wave_sum(cnt);
    if (cnt >= m) ans = cand;
  }
  return ans;
}

// "MiniMax-M3 W8A8 inference on K100AI" §3.2/§6.4: per-token symmetric INT8
// after the SmoothQuant rescaling. v_j = x_j * inv_s_j, level = max |v_j|,
// optionally lowered by a clip (§6.4: saturate instead of stretching the scale;
// "一晚上完成MoE模型推理优化…" §3.2: clip at a percentile), code =
// rint(fl32(v * fl32(127/level))) clamped to [-127, 127], scale = level/127;
// a zero level gives scale 0 and codes 0. FP8 (e4m3) codes: the same with
// 448 for 127 and f8x4 for the rounding.
// One wavefront per row; the row (H bf16) is read once, 16 bytes per lane
// per chunk, and kept in registers between the max and the code pass while
// it fits (H <= 64 * 8 * MAXC), re-read otherwise.
template <int MAXC>
__device__ __forceinline__ void quant_token_row(const uint16_t *__restrict__ xr,
                                                const float *__restrict__ inv_s, int H,
                                                int8_t *__restrict__ qr, float *__restrict__ sx,
                                                ActClip ac, bool fp8) {
  const int lane = threadIdx.x & 63;
  const int nchunk = H >> 3;
  const bool cached = nchunk <= 64 * MAXC;
  // Up to 8 chunks per lane the scaled values themselves stay in registers
  // (64 floats), so inv_s is read and multiplied once; more chunks keep the
  // raw bf16 words and scale them again when the codes are made.
  constexpr bool kKeepScaled = MAXC <= 8;
  v4i raw[MAXC];
  float sv[kKeepScaled ? MAXC : 1][8];
  float amax = 0.0f;
  auto scale8 = [&](v4i r, int c, float *o) {
    const v4f s0 = *reinterpret_cast<const v4f *>(inv_s + c * 8);
    const v4f s1 = *reinterpret_cast<const v4f *>(inv_s + c * 8 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = (uint32_t)r[i];
      const float slo = i < 2 ? s0[2 * i] : s1[2 * i - 4];
      const float shi = i < 2 ? s0[2 * i + 1] : s1[2 * i - 3];
      o[2 * i] = __uint_as_float(w << 16) * slo;
      o[2 * i + 1] = __uint_as_float(w & 0xffff0000u) * shi;
    }
  };
  if (cached) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = lane + 64 * i;
      raw[i] = c < nchunk ? *reinterpret_cast<const v4i *>(xr + c * 8) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunk) {
        float v[8];
        scale8(raw[i], c, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
          if constexpr (kKeepScaled) sv[i][j] = v[j];
        }
      }
    }
  } else {
    for (int c = lane; c < nchunk; c += 64) {
      float v[8];
      scale8(*reinterpret_cast<const v4i *>(xr + c * 8), c, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[j]));
    }
  }
  amax = wave_max(amax);
  float level = amax;
  if (ac.clip) {
    const float c = *ac.clip;
    if (c > 0.0f && c < level) level = c;
  }
  if (ac.sat_m > 1) {
    uint32_t top[kMaxSatM];
#pragma unroll
    for (int s = 0; s < kMaxSatM; ++s) top[s] = 0u;
    auto add8 = [&](v4i r, int c) {
      float v[8];
      scale8(r, c, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) top_insert(top, __float_as_uint(__builtin_fabsf(v[j])));
    };
    if (cached) {
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunk) {
          if constexpr (kKeepScaled) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              top_insert(top, __float_as_uint(__builtin_fabsf(sv[i][j])));
          } else {
            add8(raw[i], c);
          }
        }
      }
    } else {
      for (int c = lane; c < nchunk; c += 64) add8(*reinterpret_cast<const v4i *>(xr + c * 8), c);
    }
    const float t = __uint_as_float(wave_mth_largest(top, ac.sat_m, __float_as_uint(amax)));
    if (t > 0.0f && t < level) level = t;
  }
  const float qmax = fp8 ? kFp8Max : 127.0f;
  if (lane == 0) *sx = level / qmax;
  const float rr = level > 0.0f ? qmax / level : 0.0f;
  auto emit = [&](v4i r, int c) {
    float v[8];
    scale8(r, c, v);
    *reinterpret_cast<uint2 *>(qr + c * 8) = make_uint2(codes4(v, rr, fp8), codes4(v + 4, rr, fp8));
  };
  if (cached) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = lane + 64 * i;
      if (c < nchunk) {
        if constexpr (kKeepScaled)
          *reinterpret_cast<uint2 *>(qr + c * 8) =
              make_uint2(codes4(sv[i], rr, fp8), codes4(sv[i] + 4, rr, fp8));
        else
          emit(raw[i], c);
      }
    }
  } else {
    for (int c = lane; c < nchunk; c += 64) emit(*reinterpret_cast<const v4i *>(xr + c * 8), c);
  }
}

// ------------------------------------------------------------- tile order
// Tile L of a tiled GEMM's expert-major order (expert, N group, M tile, N
// tile in group) for the M-tile table mtile_off (M tiles of expert e:
// mtile_off[e] .. mtile_off[e+1]-1), nt N tiles per expert in groups of gn.
struct TileCoord {
  int e, mtl, ntile;
};
__device__ __forceinline__ TileCoord tile_coord(const int32_t *__restrict__ mtile_off, int E,
                                                int nt, int gn, int L) {
  int lo = 0, hi = E;  // largest e with mtile_off[e] * nt <= L
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mtile_off[mid] * nt <= L) lo = mid; else hi = mid;
  }
  const int mtiles = mtile_off[lo + 1] - mtile_off[lo];
  const int local = L - mtile_off[lo] * nt;
  const int grp = local / (mtiles * gn), r_in = local - grp * (mtiles * gn);
  const int mtl = r_in / gn;
  return TileCoord{lo, mtl, grp * gn + (r_in - mtl * gn)};
}

// One 256-thread block's share of GEMM g's tile order, for XCD x. With at
// most kTileOrderMaxTiles tiles:
//  - the expert-major order is cut into 8 contiguous ranges of about equal
//    estimated time (a tile of an M tile with b 64-row bands of rows costs
//    3 + b: a partial tile skips the empty bands' matrix work but still
//    streams its whole weight panel), tile j going to the XCD that holds the
//    midpoint of its cost; and
//  - XCD x runs its range sorted stably by bands (4, 3, 2, 1), so that the
//    short tiles end its queue.
// Region: order[0] flag (1: built), order[1 + x] the number of tiles of XCD
// x, order[9 + x * cap + i] its i-th tile (cap = to.cap[g], the places the
// GEMM's grid gives each XCD). Every block derives the same ranges, so the
// ones that do not fit cap (or too many tiles) leave the flag 0 everywhere.
__device__ __forceinline__ void tile_order_block(const TileOrderArgs &to, int x, int g) {
  static_assert(kTileOrderMaxTiles <= 3 * 256, "three tiles per thread");
  __shared__ int wsum[4], first[8], cnt[8];
  __shared__ int wave_n[4][4];
  int32_t *order = to.order[g];
  const int nt = to.nt[g], gn = to.gn[g], cap = to.cap[g];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = to.mtile_off[to.E] * nt;
  if (ntiles <= 0 || ntiles > kTileOrderMaxTiles) {
    if (x == 0 && tid == 0) order[0] = 0;
    return;
  }
  auto bands = [&](int L) {
    const TileCoord tc = tile_coord(to.mtile_off, to.E, nt, gn, L);
    const int rows = to.counts[tc.e] - tc.mtl * kTiledBM;
    return rows >= kTiledBM ? 4 : (rows + 63) / 64;
  };
  // costs of tiles 3t .. 3t+2 and their block-wide prefix
  int cost[3], tsum = 0;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int j = 3 * tid + s;
    cost[s] = j < ntiles ? 3 + bands(j) : 0;
    tsum += cost[s];
  }
  const int incl = wave_incl_scan(tsum);
  if (lane == 63) wsum[wave] = incl;
  if (tid < 8) {
    first[tid] = ntiles;
    cnt[tid] = 0;
  }
  __syncthreads();
  int before = incl - tsum, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  // XCD of tile j: floor(8 * (its cost midpoint) / total), monotone in j
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int j = 3 * tid + s;
    if (j < ntiles) {
      int xj = (int)((8ll * (2ll * before + cost[s])) / (2ll * total));
      xj = xj < 7 ? xj : 7;
      atomicMin(&first[xj], j);
      atomicAdd(&cnt[xj], 1);
    }
    before += cost[s];
  }
  __syncthreads();
  bool fits = true;
#pragma unroll
  for (int q = 0; q < 8; ++q) fits = fits && cnt[q] <= cap && cnt[q] <= 256;
  if (!fits) {
    if (x == 0 && tid == 0) order[0] = 0;
    return;
  }
  const int lo = first[x], len = cnt[x];
  // XCD x's tiles lo .. lo+len-1, stably by bands, most first
  int c = 4;  // no tile
  if (tid < len) c = 4 - bands(lo + tid);
  int rank = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t m = __ballot(c == q);
    if (c == q) rank = __builtin_popcountll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wave_n[wave][q] = __builtin_popcountll(m);
  }
  __syncthreads();
  if (c < 4) {
    int pos = rank;
    for (int q = 0; q < c; ++q)
      for (int w = 0; w < 4; ++w) pos += wave_n[w][q];
    for (int w = 0; w < wave; ++w) pos += wave_n[w][c];
    order[9 + x * cap + pos] = lo + tid;
  }
  if (tid == 0) {
    order[1 + x] = len;
    if (x == 0) order[0] = 1;
  }
}

// ------------------------------------------------------------------ combine
// "超大规模模型推理的Day0适配实践" §四: un-sort and gate-weighted sum of token t:
//   out[t][n] = bf16( sum over slots j < k with row_of[t*k+j] >= 0 of
//                     w[t][j] * y[row][n] )
// summed in fp32 in slot order (independent of scheduling), bf16 with ties
// to even. Dropped slots add nothing; the remaining weights are not
// renormalised. Callers place the groups of a wavefront's 64 lanes so that
// each load instruction reads 1 KB of one y row.
//
// combine_2x4: fp32 y rows; two groups of four consecutive outputs at n0
// and n1 (a group at or past H is skipped; H is a multiple of 4).
__device__ __forceinline__ void combine_2x4(const float *__restrict__ y,
                                            const float *__restrict__ wts,
                                            const int32_t *__restrict__ row_of, int64_t t, int H,
                                            int k, int n0, int n1, uint16_t *__restrict__ out) {
  const bool g0 = n0 < H, g1 = n1 < H;
  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  // Slots 8 at a time: all loads of a batch are issued before the sums,
  // which then run in slot order over the kept slots.
  for (int j0 = 0; j0 < k; j0 += 8) {
    v4f v0[8], v1[8];
    float w[8];
    bool kept[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      const int32_t r = j < k ? row_of[t * k + j] : -1;
      kept[u] = r >= 0;
      w[u] = kept[u] ? wts[t * k + j] : 0.0f;
      if (kept[u]) {
        const float *yr = y + (int64_t)r * H;
        if (g0) v0[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(yr + n0));
        if (g1) v1[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(yr + n1));
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (!kept[u]) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc0[i] += w[u] * v0[u][i];
        acc1[i] += w[u] * v1[u][i];
      }
    }
  }
  v2i o0, o1;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    o0[i] = (int)((uint32_t)f32_to_bf16(acc0[2 * i]) | ((uint32_t)f32_to_bf16(acc0[2 * i + 1]) << 16));
    o1[i] = (int)((uint32_t)f32_to_bf16(acc1[2 * i]) | ((uint32_t)f32_to_bf16(acc1[2 * i + 1]) << 16));
  }
  if (g0) *reinterpret_cast<v2i *>(out + t * H + n0) = o0;
  if (g1) *reinterpret_cast<v2i *>(out + t * H + n1) = o1;
}

// combine_2x8: y rows as int16 codes with a scale per 16 columns (YRows,
// y[row][n] = fl32(code * scale)); two groups of eight consecutive outputs
// at n0 and n1 (multiples of 8; a group at or past H is skipped).
__device__ __forceinline__ void combine_2x8(const YRows y, const float *__restrict__ wts,
                                            const int32_t *__restrict__ row_of, int64_t t, int H,
                                            int k, int n0, int n1, uint16_t *__restrict__ out) {
  const bool g0 = n0 < H, g1 = n1 < H;
  const int64_t hg = H / kYGroup;
  float acc0[8], acc1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc0[i] = acc1[i] = 0.0f;
  // Slots 8 at a time: all loads of a batch are issued before the sums,
  // which then run in slot order over the kept slots.
  for (int j0 = 0; j0 < k; j0 += 8) {
    v4i c0[8], c1[8];
    float s0[8], s1[8], w[8];
    bool kept[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      const int32_t r = j < k ? row_of[t * k + j] : -1;
      kept[u] = r >= 0;
      w[u] = kept[u] ? wts[t * k + j] : 0.0f;
      if (kept[u]) {
        const int16_t *yr = y.q + (int64_t)r * H;
        const float *sr = y.s + (int64_t)r * hg;
        if (g0) {
          c0[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(yr + n0));
          s0[u] = sr[n0 / kYGroup];
        }
        if (g1) {
          c1[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(yr + n1));
          s1[u] = sr[n1 / kYGroup];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (!kept[u]) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // code i of the group: low half of word i/2 for even i, high half for odd
        const int wd0 = c0[u][i >> 1], wd1 = c1[u][i >> 1];
        const float q0 = (float)((i & 1) ? (wd0 >> 16) : (int)(int16_t)wd0);
        const float q1 = (float)((i & 1) ? (wd1 >> 16) : (int)(int16_t)wd1);
        acc0[i] += w[u] * (q0 * s0[u]);
        acc1[i] += w[u] * (q1 * s1[u]);
      }
    }
  }
  v4i o0, o1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o0[i] = (int)((uint32_t)f32_to_bf16(acc0[2 * i]) | ((uint32_t)f32_to_bf16(acc0[2 * i + 1]) << 16));
    o1[i] = (int)((uint32_t)f32_to_bf16(acc1[2 * i]) | ((uint32_t)f32_to_bf16(acc1[2 * i + 1]) << 16));
  }
  if (g0) *reinterpret_cast<v4i *>(out + t * H + n0) = o0;
  if (g1) *reinterpret_cast<v4i *>(out + t * H + n1) = o1;
}

}  // namespace moe
