// gemm_tiled.hip -- grouped INT8 GEMMs for many rows per expert (prefill).
//
// "MiniMax-M3 W8A8 inference on K100AI" (mhpq.cn/news/1068415) §1.1/§4.3:
// batch-level scheduling so that expert compute is one large grouped GEMM
// rather than many small ones; §1.2: INT8 x INT8 with integer accumulation,
// dequantised afterwards; "一晚上完成MoE模型推理优化…" §4.1: the activation
// that follows a linear layer is fused into it (SwiGLU in GEMM1's epilogue).
// FP8 codes ("超大规模模型推理的Day0适配实践" §二.1, §四) use the same tiles and
// pipeline: the two 32-byte k halves of a stage feed one
// v_mfma_scale_f32_32x32x64_f8f6f4 with fp32 accumulators.
//
// One block (8 wavefronts, two per SIMD) computes a 256-row x 384-column
// tile of one expert:
//   rows    = 256 consecutive permuted rows of the expert (the M tile);
//   columns = GEMM1: 192 gate channels and the same 192 up channels of the
//             expert's [2F][H] weights; GEMM2: 384 output channels. The last
//             N tile of an expert may be partial (F a multiple of 32, H of
//             256): its missing weight tiles repeat the last real one and
//             their columns are not stored.
// Operands reach LDS through direct global->LDS loads (global_load_lds_dwordx4:
// one instruction moves 1 KB, lane l's 16 bytes landing at byte 16*l), with
// all 160 KB of LDS as rings of stages. The weights, and GEMM2's activations,
// are stored fragment-tiled (16 rows x 64 k per 1 KB, the lane order of the
// INT8 matrix instructions; by calibration and by the requantisation, expert
// groups starting on a 16-row boundary) and move as whole tiles; reading a
// 32x32x32 operand from such a tile is a conflict-free ds_read_b128. GEMM2
// runs one ring of four 64-k stages of 40 KB, three ahead. GEMM1's
// activations are gathered by the loads themselves from the token-major
// codes, so every token row is read where it lies (T x H bytes, which stay
// cache-resident across the k experts that use them) instead of from a
// permuted copy k times that size: they come through their own ring of two
// 128-k stages, each lane fetching 16 bytes so that one instruction reads
// whole 128-byte lines of eight token rows, into an XOR-swizzled row-major
// layout, beside a ring of four 64-k weight stages.
// What limits these kernels is the operand feed, about 14 B per clock per CU
// at prefill: a stage waits for its slowest line, and the 16-23 % of lines
// that miss L2 come from the last-level cache or HBM. (One block per CU can
// move ~49 B per clock into LDS when every line hits L2.) The tile is
// therefore as large as the registers allow: 256 x 384 moves 40 KB per
// 6.3 M multiply-adds, a fifth less per operation than 256 x 256.
// Wavefront (wm, wn), wm < 4, wn < 2, owns rows 64*wm.. and six 32-column
// fragments: for GEMM1 three gate and the three matching up fragments (so g
// and u of one h element meet in one lane), for GEMM2 192 consecutive
// outputs; it accumulates a 64x192 tile in 12 32x32 accumulators
// (v_mfma_i32_32x32x32_i8). The epilogue goes through the wavefront's own
// slice of the (then free) stage buffers so that every global store writes
// 16 bytes per lane along a row.
//
// Tiles are numbered expert by expert, and within an expert (N group, M tile,
// N tile in group), so that the blocks that run together on one XCD (one L2)
// share a few weight panels and reuse each activation tile across the group;
// each XCD takes one contiguous eighth of that order. When a GEMM has at
// most three rounds of tiles, the order built by tile_order_block (in the
// scatter launch) is used instead: contiguous ranges of equal estimated
// time per XCD, each run longest first. A tile of a group's last, partial
// M tile skips the matrix work of its empty 64-row bands and takes up to
// ~40 % less time, so these end the XCD's queue instead of a few long tiles
// holding up a mostly idle last round. With more rounds the blocks that
// finish at different times already keep the compute units busy, and the
// expert-major order keeps a partial M tile's weight panels in the caches.
// The grid gives each XCD as many places as either order can need; surplus
// blocks exit at once.
#include <type_traits>

#include "layer_device.h"

// The direct-to-LDS loads are issued from inline assembly: the compiler's own
// intrinsic makes every later LDS read wait for all outstanding loads, which
// would drain the stage ring on each step. The assembly sets M0 (the LDS base
// of the wavefront's 1 KB) itself, and the waits are explicit below.
#pragma clang diagnostic ignored "-Winline-asm"

namespace moe {
namespace {

constexpr int BM = kTiledBM;  // 256 rows
constexpr int BN = 384;       // output columns (GEMM1: 192 gate + 192 up)
constexpr int BK = 64;        // k bytes per stage
constexpr int kStages = 4;
constexpr int kWaves = 8;
constexpr int kATiles = BM / 16, kBTiles = BN / 16;      // 1 KB tiles per stage
constexpr int kStageBytes = (kATiles + kBTiles) * 1024;  // 40 KB
constexpr int kALoads = kATiles / kWaves, kBLoads = kBTiles / kWaves;
constexpr int kLoadsPerWave = kALoads + kBLoads;         // 2 + 3
static_assert(kALoads * kWaves == kATiles && kBLoads * kWaves == kBTiles, "load split");
// Epilogue staging: 32 rows x 96 columns per pass, row pitch padded by 8
// floats so that the two 32-lane halves of a wavefront (rows r and r+4) use
// disjoint banks.
constexpr int kEpiPitch = 96 + 8;
constexpr int kSlice = 32 * kEpiPitch * 4;    // per-wavefront epilogue staging
constexpr int kRowScaleAt = kWaves * kSlice;  // then 256 row scales
// GEMM2 stages 16 rows x 192 columns per pass (the same pitch rule).
constexpr int kEpiPitch2 = 192 + 8;
constexpr int kSlice2 = 16 * kEpiPitch2 * 4;
static_assert(kSlice2 <= kSlice, "GEMM2 epilogue staging");
// After the row scales: per wavefront, GEMM2's 16 x 12 group scales of a
// pass, stored by one instruction (16 bytes per lane).
constexpr int kScaleStageAt = kRowScaleAt + BM * 4;
static_assert(kScaleStageAt + kWaves * 16 * 12 * 4 <= kStages * kStageBytes, "epilogue staging");
static_assert(kRowScaleAt + BM * 4 <= kStages * kStageBytes, "epilogue staging");
static_assert(kEpiPitch > 96, "GEMM1 keeps each staged row's maximum in column 96");

struct TiledArgs {
  const int8_t *act;        // GEMM1: token-major codes [T][K]; GEMM2: fragment-tiled
                            // padded rows [rows/16][K/64] x 1 KB
  const float *row_scale;   // GEMM1: per token (sx); GEMM2: per padded row (sh)
  const int32_t *gather;    // GEMM1: assignment t*k+j of each padded row, -1 if padding
  int topk;
  const int32_t *counts, *offsets, *mtile_off;  // offsets: 16-aligned group starts
  const int32_t *dense_off;                     // GEMM1: dense group starts (debug rows)
  int E;
  int nt;                   // N tiles per expert
  int gn;                   // N tiles per group (divides nt)
  const int32_t *order;     // tile order region (see tile_order_block), or NULL
  int places;               // places per XCD in the grid (the region's stride)
  const int8_t *w;          // fragment-tiled weights
  const float *wscale;
  int K, F, H;
  float *out;               // GEMM1: h [rows][F]
  YRows y;                  // GEMM2: y rows (int16 codes, a scale per 16 columns)
  uint32_t *amax;           // GEMM1: row max |h| (float bits)
  int32_t *acc1_dbg;        // GEMM1: optional INT32 accumulators, dense rows [A][2F]
};

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void *)p);
}
// 16 bytes per lane from global memory into LDS at lds_base + 16*lane. An
// LDS-DMA load needs one wait state after M0 is written.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}
// Wait until at most N of this wavefront's loads are in flight and its LDS
// accesses are done, then meet the other wavefronts of the block.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Maximum of a non-negative value over each 32-lane half of the wavefront,
// by DPP moves (no LDS round trip): row_shr 1, 2, 4, 8 leave each 16-lane
// row's maximum in its lane 15, and row_bcast15 into rows 1 and 3 adds the
// row below. The results land in lanes 31 and 63. Non-negative floats order
// as their bit patterns, so the maximum is taken on those.
__device__ __forceinline__ uint32_t half_wave_max(uint32_t m) {
  auto step = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
  m = step(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x111, 0xF, 0xF, false));
  m = step(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x112, 0xF, 0xF, false));
  m = step(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x114, 0xF, 0xF, false));
  m = step(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x118, 0xF, 0xF, false));
  m = step(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x142, 0xA, 0xF, false));
  return m;
}

// silu(g) * u with the hardware exponential and reciprocal.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Accumulators: INT32 for INT8 codes, fp32 for FP8 codes.
template <bool kF8> struct Acc32 { typedef v16i T; };
template <> struct Acc32<true> { typedef v16f T; };

template <bool kGateUp, bool kF8>
__global__ __launch_bounds__(512, 1) void gemm_tiled_kernel(const TiledArgs a) {
  typedef typename Acc32<kF8>::T Acc;
  // All 160 KB: the operand rings (GEMM2: four 40 KB stages; GEMM1: two
  // 32 KB activation stages and four 24 KB weight stages), then (after the
  // K loop) the epilogue staging and the row scales.
  __shared__ __attribute__((aligned(1024))) int8_t lds[kStages * kStageBytes];
  float *row_scale = reinterpret_cast<float *>(lds + kRowScaleAt);

  // Tiles in expert-major order (expert, N group, M tile, N tile in group),
  // cut into 8 equal contiguous chunks of the actual tile count, chunk x on
  // XCD x (blocks are dealt to the XCDs round-robin by id). An XCD thus runs
  // an expert's N groups back to back: the expert's weights are read once
  // and its activation tiles are re-read while still in the caches.
  const int E = a.E;
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int ntiles = a.mtile_off[E] * a.nt;
  int L;
  if (a.order && a.order[0]) {
    // the XCD's range of the tile order (equal estimated time, longest first)
    if (idx >= a.order[1 + xcd]) return;
    L = a.order[9 + xcd * a.places + idx];
  } else {
    const int chunk = (ntiles + 7) >> 3;
    if (idx >= chunk) return;
    L = xcd * chunk + idx;
  }
  if (L < 0 || L >= ntiles) return;
  const TileCoord tc = tile_coord(a.mtile_off, E, a.nt, a.gn, L);
  const int e = tc.e, mtl = tc.mtl, ntile = tc.ntile;
  const int R = a.counts[e];
  const int row0 = a.offsets[e];  // multiple of 16
  const int m0 = mtl * BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.K, F = a.F, H = a.H;
  const int KT = K / BK;

  const int N = kGateUp ? 2 * F : H;
  const int8_t *wexp = a.w + (size_t)e * (size_t)N * (size_t)K;
  const int last_rt = (row0 + R - 1) >> 4;
  // In the last, partial M tile of a group, a wavefront whose 32 activation
  // load rows (32w..32w+31) all lie past the group issues no activation loads,
  // and one whose 64 compute rows (64wm..) all do skips its matrix work; the
  // stale LDS rows they leave only meet rows that are never stored.
  const bool skip_a = m0 + 32 * wave >= R;
  const bool skip_mma = m0 + 64 * wm >= R;

  // Weight tiles 3w .. 3w+2 of each stage are this wavefront's loads. Tiles
  // past the last channel repeat it (their columns are never stored).
  const int8_t *bsrc[kBLoads];
  int bdst[kBLoads];
#pragma unroll
  for (int t = 0; t < kBLoads; ++t) {
    const int bi = kBLoads * wave + t;
    int wt;  // 16-channel weight tile
    if (kGateUp) {
      const int half = bi / 12, j = ntile * 12 + bi % 12;  // gate (0) or up (1)
      wt = half * (F >> 4) + (j < (F >> 4) ? j : (F >> 4) - 1);
    } else {
      const int j = ntile * 24 + bi;
      wt = j < (H >> 4) ? j : (H >> 4) - 1;
    }
    bsrc[t] = wexp + frag_tile(wt, 0, K) + lane * 16;
    bdst[t] = bi * 1024;
  }

  Acc acc[2][6];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < 6; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][c][v] = 0;

  // Weight operand offsets inside a stage's weight tiles: the 32x32x32
  // fragment of column block c, k half 0, starts in tile t0 + (lane%32)/16 at
  // lane row lane%16, k group lane/32 (k half 1: + 512).
  const int frag = (((lane >> 5) * 16) + (lane & 15)) * 16 + ((lane & 31) >> 4) * 1024;
  int boff[6];
#pragma unroll
  for (int c = 0; c < 6; ++c) {
    const int t0 = kGateUp ? (c < 3 ? 6 * wn + 2 * c : 12 + 6 * wn + 2 * (c - 3))
                           : 12 * wn + 2 * c;
    boff[c] = t0 * 1024 + frag;
  }

  // One 64-k step of matrix work: A fragment (row block i, k half hk) at
  // ap[i][hk], the weight tiles of the stage at bst.
  auto step = [&](const int8_t *const (&ap)[2][2], const int8_t *bst) {
    v4i af[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) af[i][hk] = *reinterpret_cast<const v4i *>(ap[i][hk]);
    // The next column fragment's halves are read while the current one's
    // instructions run.
    v4i b0 = *reinterpret_cast<const v4i *>(bst + boff[0]);
    v4i b1 = *reinterpret_cast<const v4i *>(bst + boff[0] + 512);
#pragma unroll
    for (int c = 0; c < 6; ++c) {
      v4i n0 = b0, n1 = b1;
      if (c < 5) {
        n0 = *reinterpret_cast<const v4i *>(bst + boff[c + 1]);
        n1 = *reinterpret_cast<const v4i *>(bst + boff[c + 1] + 512);
      }
      if constexpr (kF8) {
        // both k halves feed one 32x32x64 FP8 instruction
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][c] = mfma32f8(af[i][0], af[i][1], b0, b1, acc[i][c]);
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][c] = mfma32(af[i][0], b0, acc[i][c]);
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][c] = mfma32(af[i][1], b1, acc[i][c]);
      }
      b0 = n0; b1 = n1;
    }
    // Issue order: the A halves and two column fragments, then per fragment
    // its instructions followed by the reads of the fragment two ahead, so
    // one fragment's reads are always in flight.
    constexpr int kM = kF8 ? 2 : 4;  // instructions per column fragment
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      __builtin_amdgcn_sched_group_barrier(0x008, kM, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kM, 0);
  };

  if constexpr (kGateUp) {
    // GEMM1. The gathered activation rows come through a ring of two
    // 128-k "double stages" (32 KB each: 256 rows x 128 bytes), so that each
    // load instruction reads whole 128-byte lines of eight token rows; the
    // weights through a ring of four 64-k stages (24 KB each). Chunk c (16 bytes) of
    // row r sits at r*128 + 16*(c ^ ((r/2)%8)): any 16 consecutive rows then
    // put one chunk in 16 distinct 16-byte bank groups of a 256-byte line,
    // so a matrix operand read is conflict-free. Instruction q of a double
    // stage fills rows 8q..8q+7 (lane l: row 8q + l/8, slot l%8, byte 16*l).
    constexpr int kA2 = BM * 128;                 // one double stage
    constexpr int kBStage = kBTiles * 1024;       // one weight stage
    static_assert(2 * kA2 + 4 * kBStage <= kStages * kStageBytes, "GEMM1 rings");
    const int8_t *asrc[4];
    int adst[4];
    const int last_p = last_rt * 16 + 15;  // last padded row of the expert
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int q = 4 * wave + t;
      int p = row0 + m0 + 8 * q + (lane >> 3);
      p = p < last_p ? p : last_p;  // rows past the expert: computed, never stored
      const int asg = a.gather[p];
      const int64_t tok = asg >= 0 ? asg / a.topk : 0;  // padding rows read token 0
      // the chunk that belongs in slot l%8 of row 8q + l/8
      asrc[t] = a.act + tok * K + (((lane & 7) ^ ((4 * (q & 1) + (lane >> 4)) & 7)) << 4);
      adst[t] = q * 1024;
    }
    auto issue_a = [&](int d) {
      int8_t *st = lds + (d & 1) * kA2;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        dma16(asrc[t] + (size_t)d * 128, __builtin_amdgcn_readfirstlane(lds_addr(st + adst[t])));
    };
    auto issue_b = [&](int kt) {
      int8_t *st = lds + 2 * kA2 + (kt & 3) * kBStage;
#pragma unroll
      for (int t = 0; t < kBLoads; ++t)
        dma16(bsrc[t] + ((size_t)kt << 10), __builtin_amdgcn_readfirstlane(lds_addr(st + bdst[t])));
    };
    // A operand byte offsets: row 64*wm + 32*i + lane%32, chunk
    // 4*(kt%2) + 2*hk + lane/32, swizzled by (row/2)%8 = (lane/2)%8.
    int arow[2], axor[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) arow[i] = (64 * wm + 32 * i + (lane & 31)) * 128;
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
      for (int hk = 0; hk < 2; ++hk)
        axor[par][hk] = ((4 * par + 2 * hk + (lane >> 5)) ^ ((lane >> 1) & 7)) << 4;
    // Issue order (K / 64 = KT steps, even): B(0); A(0), B(1); B(2); then at
    // step kt, after the wait, A(kt/2 + 1) on even kt and B(kt + 3). Waiting
    // at step kt for B(kt) (and on even kt for A(kt/2)) leaves 6 loads in
    // flight on even kt and 10 on odd kt; the last three steps drain all.
    // A wavefront without activation loads waits for B(kt) alone: two B
    // stages in flight on every step.
    issue_b(0);
    if (!skip_a) issue_a(0);
    issue_b(1);
    issue_b(2);
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 3 < KT) {
        if ((kt & 1) && !skip_a) wait_barrier<2 * kBLoads + 4>();
        else wait_barrier<2 * kBLoads>();
      } else {
        wait_barrier<0>();
      }
      if (!skip_a && !(kt & 1) && 2 * (kt / 2 + 1) < KT) issue_a(kt / 2 + 1);
      if (kt + 3 < KT) issue_b(kt + 3);
      const int8_t *as = lds + ((kt >> 1) & 1) * kA2;
      const int par = kt & 1;
      const int8_t *ap[2][2] = {{as + arow[0] + axor[par][0], as + arow[0] + axor[par][1]},
                                {as + arow[1] + axor[par][0], as + arow[1] + axor[par][1]}};
      if (!skip_mma) step(ap, lds + 2 * kA2 + (kt & 3) * kBStage);
    }
  } else {
    // GEMM2: both operands fragment-tiled, one ring of four 64-k stages of
    // 40 KB (16 activation tiles, then 24 weight tiles); this wavefront loads
    // activation tiles 2w, 2w+1 (clamped to the expert's last row tile:
    // their rows are computed and never stored) and its weight tiles, three
    // stages ahead.
    const int8_t *asrc[kALoads];
    int adst[kALoads];
#pragma unroll
    for (int t = 0; t < kALoads; ++t) {
      const int ti = kALoads * wave + t;
      int rt = ((row0 + m0) >> 4) + ti;
      rt = rt < last_rt ? rt : last_rt;
      asrc[t] = a.act + frag_tile(rt, 0, K) + lane * 16;
      adst[t] = ti * 1024;
    }
    // A operand: row block 32 of tile 4*wm + 2*i, as for the weights.
    const int aoff = (4 * wm) * 1024 + frag;
    const int pre = KT < kStages - 1 ? KT : kStages - 1;
    auto kloop = [&](auto skip) {
      constexpr bool kSkipA = decltype(skip)::value;
      constexpr int kLoads = kSkipA ? kBLoads : kLoadsPerWave;  // per stage and wavefront
      auto issue = [&](int kt) {
        int8_t *st = lds + (kt % kStages) * kStageBytes;
        if (!kSkipA) {
#pragma unroll
          for (int t = 0; t < kALoads; ++t)
            dma16(asrc[t] + ((size_t)kt << 10),
                  __builtin_amdgcn_readfirstlane(lds_addr(st + adst[t])));
        }
#pragma unroll
        for (int t = 0; t < kBLoads; ++t)
          dma16(bsrc[t] + ((size_t)kt << 10),
                __builtin_amdgcn_readfirstlane(lds_addr(st + kATiles * 1024 + bdst[t])));
      };
      for (int s2 = 0; s2 < pre; ++s2) issue(s2);
      for (int kt = 0; kt < KT; ++kt) {
        const int ahead = KT - 1 - kt < kStages - 2 ? KT - 1 - kt : kStages - 2;
        static_assert(kStages - 2 <= 2, "wait cases");
        if (ahead >= 2) wait_barrier<2 * kLoads>();
        else if (ahead == 1) wait_barrier<kLoads>();
        else wait_barrier<0>();
        if (kt + kStages - 1 < KT) issue(kt + kStages - 1);
        const int8_t *st = lds + (kt % kStages) * kStageBytes;
        const int8_t *ap[2][2] = {{st + aoff, st + aoff + 512},
                                  {st + aoff + 2048, st + aoff + 2048 + 512}};
        if (!skip_mma) step(ap, st + kATiles * 1024);
      }
    };
    if (skip_a) kloop(std::true_type{});
    else kloop(std::false_type{});
  }
  // Every wavefront is done with the stage buffers before they are reused.
  wait_barrier<0>();
  if (tid < BM) {
    const int r = m0 + tid;
    float sc = 0.0f;
    if (r < R) sc = kGateUp ? a.row_scale[a.gather[row0 + r] / a.topk] : a.row_scale[row0 + r];
    row_scale[tid] = sc;
  }
  __syncthreads();

  // Epilogue, 32 rows (row block i) at a time through this wavefront's LDS
  // slice. Lane holds column (lane & 31) of each 32x32 accumulator tile and
  // rows 8*(v/4) + 4*(lane/32) + v%4, v < 16.
  float *slice = reinterpret_cast<float *>(lds + wave * kSlice);
  const int mw = 64 * wm;
  const int rl = 4 * (lane >> 5);  // lane's row offset inside a group of 8
  if (kGateUp) {
    const int f0 = ntile * 192 + 96 * wn;  // first h column of this wavefront
    const float *sgu = a.wscale + (size_t)e * 2 * F;
    // Columns past F (a partial last tile) get zero scales: their h is 0
    // and leaves the row maxima alone.
    float sg[3], su[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const int f = f0 + 32 * c + (lane & 31);
      sg[c] = f < F ? sgu[f] : 0.0f;
      su[c] = f < F ? sgu[F + f] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      // The scales of the lane's 16 rows (four runs of 4 consecutive rows),
      // read before the pass's staging writes: a read issued after them
      // cannot be moved ahead (the compiler cannot rule out aliasing) and
      // waits for every write before it.
      v4f rsc[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        rsc[g] = *reinterpret_cast<const v4f *>(row_scale + mw + 32 * i + 8 * g + rl);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + rl + (v & 3);
        const float sxv = rsc[v >> 2][v & 3];
        float mx = 0.0f;
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          const float hv = swiglu((float)acc[i][c][v] * sxv * sg[c],
                                  (float)acc[i][3 + c][v] * sxv * su[c]);
          slice[r * kEpiPitch + 32 * c + (lane & 31)] = hv;
          mx = __builtin_fmaxf(mx, __builtin_fabsf(hv));
        }
        // row maximum over the wavefront's 96 columns (the 32 lanes of a
        // half), taken by lanes 31 and 63 into the slice's padding column
        // 96 (the passes write columns 0..95 only)
        const uint32_t mb = half_wave_max(__float_as_uint(mx));
        if ((lane & 31) == 31) slice[r * kEpiPitch + 96] = __uint_as_float(mb);
      }
      if (a.acc1_dbg) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = mw + 32 * i + 8 * (v >> 2) + rl + (v & 3);
          if (m0 + m >= R) continue;
          const size_t row = (size_t)(a.dense_off[e] + m0 + m);
#pragma unroll
          for (int c = 0; c < 3; ++c) {
            const int f = f0 + 32 * c + (lane & 31);
            if (f < F) {
              // The element is copied out before its bits are taken: a bit
              // cast applied to a vector element directly reads element 0.
              const auto gv = acc[i][c][v], uv = acc[i][3 + c][v];
              a.acc1_dbg[row * 2 * F + f] = __builtin_bit_cast(int32_t, gv);
              a.acc1_dbg[row * 2 * F + F + f] = __builtin_bit_cast(int32_t, uv);
            }
          }
        }
      }
      // the 32 row maxima by one atomic instruction (order independent)
      if (lane < 32 && m0 + mw + 32 * i + lane < R)
        atomicMax(a.amax + row0 + m0 + mw + 32 * i + lane,
                  __float_as_uint(slice[lane * kEpiPitch + 96]));
      // 32 rows x 96 columns: 24 lanes per row, 4 floats each; all reads
      // are issued before the first store.
      v4f hq[12];
#pragma unroll
      for (int j = 0; j < 12; ++j) {
        const int c = j * 64 + lane;
        hq[j] = *reinterpret_cast<const v4f *>(slice + (c / 24) * kEpiPitch + (c % 24) * 4);
      }
#pragma unroll
      for (int j = 0; j < 12; ++j) {
        const int c = j * 64 + lane;
        const int r = c / 24, c4 = (c % 24) * 4;
        const int m = mw + 32 * i + r;
        if (m0 + m < R && f0 + c4 < F)
          __builtin_nontemporal_store(
              hq[j], reinterpret_cast<v4f *>(a.out + (size_t)(row0 + m0 + m) * F + f0 + c4));
      }
    }
  } else {
    const int n0 = ntile * 384 + 192 * wn;  // first y column of this wavefront
    float sd[6];
#pragma unroll
    for (int c = 0; c < 6; ++c) {
      const int n = n0 + 32 * c + (lane & 31);
      sd[c] = n < H ? a.wscale[(size_t)e * H + n] : 0.0f;
    }
    // this wavefront's 12 column groups (16 columns each) start at group g0
    // of a row; a pass's 16 x 12 scales are staged in LDS
    const int hg = H / kYGroup, g0 = n0 / kYGroup;
    float *sstage = reinterpret_cast<float *>(lds + kScaleStageAt) + 16 * 12 * wave;
    float *slice2 = reinterpret_cast<float *>(lds + wave * kSlice2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      // the lane's 16 row scales, read ahead of the staging writes (as above)
      v4f rsc[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        rsc[g] = *reinterpret_cast<const v4f *>(row_scale + mw + 32 * i + 8 * g + rl);
      // Two passes of 16 rows x the wavefront's 192 columns: rows 16*vh..
      // 16*vh+15 of row block i are the lane's v = 8*vh..8*vh+7, and each
      // pass stores whole 384-byte runs of code rows.
#pragma unroll
      for (int vh = 0; vh < 2; ++vh) {
#pragma unroll
        for (int vv = 0; vv < 8; ++vv) {
          const int v = 8 * vh + vv;
          const int r = 8 * (vv >> 2) + rl + (v & 3);  // row within the pass
          const float shv = rsc[v >> 2][v & 3];
#pragma unroll
          for (int c = 0; c < 6; ++c)
            slice2[r * kEpiPitch2 + 32 * c + (lane & 31)] = (float)acc[i][c][v] * shv * sd[c];
        }
        // 16 rows x 192 columns: 24 lanes per row, 8 floats each, so that
        // every lane stores 16 bytes of codes; the two lanes 2g, 2g+1 of a
        // row hold one 16-column group (groups start on multiples of 16
        // columns), which takes one scale. All twelve staging reads come
        // before the first store.
        v4f yq[6][2];
#pragma unroll
        for (int j = 0; j < 6; ++j) {
          const int c = j * 64 + lane;
          const float *src = slice2 + (c / 24) * kEpiPitch2 + (c % 24) * 8;
          yq[j][0] = *reinterpret_cast<const v4f *>(src);
          yq[j][1] = *reinterpret_cast<const v4f *>(src + 4);
        }
#pragma unroll
        for (int j = 0; j < 6; ++j) {
          const int c = j * 64 + lane;
          const int r = c / 24, c8 = (c % 24) * 8;
          const int m = mw + 32 * i + 16 * vh + r;
          const v4f ya = yq[j][0], yb = yq[j][1];
          float gm = 0.0f;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            gm = __builtin_fmaxf(gm, __builtin_fmaxf(__builtin_fabsf(ya[q]), __builtin_fabsf(yb[q])));
          // the neighbour lane's maximum by a DPP quad permutation (1,0,3,2)
          gm = __builtin_fmaxf(gm, __int_as_float(__builtin_amdgcn_update_dpp(
                                       0, __float_as_int(gm), 0xB1, 0xF, 0xF, false)));
          if (m0 + m < R && n0 + c8 < H) {
            const size_t row = (size_t)(row0 + m0 + m);
            const float inv = y16_inv(gm);
            const v4i q = {y16x2(ya[0], ya[1], inv), y16x2(ya[2], ya[3], inv),
                           y16x2(yb[0], yb[1], inv), y16x2(yb[2], yb[3], inv)};
            __builtin_nontemporal_store(q, reinterpret_cast<v4i *>(a.y.q + row * H + n0 + c8));
          }
          // every group's scale (0 for rows and columns that are not stored)
          if ((lane & 1) == 0) sstage[r * 12 + c8 / kYGroup] = y16_scale(gm);
        }
        // The pass's scales by one instruction: lane l < 48 stores groups
        // 4(l%3)..4(l%3)+3 of row l/3 (16 bytes). The 16 rows are a 16-row
        // block of the expert's padded group whenever the block starts
        // before R (their padding rows get scale 0); groups at or past H/16
        // (a partial last N tile) are not stored.
        const int mb0 = m0 + mw + 32 * i + 16 * vh;
        const int gq = g0 + 4 * (lane % 3);
        if (lane < 48 && mb0 < R && gq < hg)
          *reinterpret_cast<v4f *>(a.y.s + (size_t)(row0 + mb0 + lane / 3) * hg + gq) =
              *reinterpret_cast<const v4f *>(sstage + 4 * lane);
      }
    }
  }
}

// N tiles per L2 group: the largest divisor of nt that is at most 4.
int group_n(int nt) {
  for (int g = 4; g > 1; --g)
    if (nt % g == 0) return g;
  return 1;
}
int gemm1_ntiles(int F) { return (F + 191) / 192; }
int gemm2_ntiles(int H) { return (H + BN - 1) / BN; }
int64_t mtile_bound(int64_t A, int E) { return (A + BM - 1) / BM + E; }
// places per XCD in a tiled GEMM's grid
int xcd_places(int64_t A, int E, int nt) {
  const int64_t p = (mtile_bound(A, E) * nt + 7) / 8;
  return (int)(p > kTileOrderPlaces ? p : kTileOrderPlaces);
}

}  // namespace

size_t tile_order_ints(int64_t A, int E, int F, int H) {
  return 18 + 8 * (size_t)(xcd_places(A, E, gemm1_ntiles(F)) + xcd_places(A, E, gemm2_ntiles(H)));
}

// GEMM1's region first (flag, 8 counts, 8 x places tiles), then GEMM2's.
TileOrderArgs tile_order_args(int64_t A, int E, int F, int H, const int32_t *counts,
                              const int32_t *mtile_off, int32_t *region) {
  TileOrderArgs to{};
  to.counts = counts; to.mtile_off = mtile_off; to.E = E;
  to.nt[0] = gemm1_ntiles(F); to.gn[0] = group_n(to.nt[0]);
  to.nt[1] = gemm2_ntiles(H); to.gn[1] = group_n(to.nt[1]);
  to.cap[0] = xcd_places(A, E, to.nt[0]);
  to.cap[1] = xcd_places(A, E, to.nt[1]);
  if (region) {
    to.order[0] = region;
    to.order[1] = region + 9 + 8 * (size_t)to.cap[0];
  }
  return to;
}

hipError_t launch_gemm1_tiled(const int8_t *qx, const float *sx, const int32_t *sorted, int k,
                              const int32_t *counts, const int32_t *offsets,
                              const int32_t *dense_off, const int32_t *mtile_off,
                              const int32_t *order, int64_t A, const int8_t *w_gu,
                              const float *s_gu, int H, int F, int E, float *h, uint32_t *amax,
                              int32_t *acc1_dbg, bool fp8, hipStream_t st, Timing tm) {
  TiledArgs a{};
  a.act = qx; a.row_scale = sx; a.gather = sorted; a.topk = k; a.counts = counts;
  a.offsets = offsets; a.dense_off = dense_off; a.mtile_off = mtile_off; a.E = E;
  a.order = order;
  a.nt = gemm1_ntiles(F); a.gn = group_n(a.nt);
  a.places = xcd_places(A, E, a.nt);
  a.w = w_gu; a.wscale = s_gu; a.K = H; a.F = F; a.H = H; a.out = h; a.amax = amax;
  a.acc1_dbg = acc1_dbg;
  const dim3 grid((unsigned)(8 * a.places));
  if (fp8) return launch_kernel(gemm_tiled_kernel<true, true>, grid, dim3(512), st, tm, a);
  return launch_kernel(gemm_tiled_kernel<true, false>, grid, dim3(512), st, tm, a);
}

hipError_t launch_gemm2_tiled(const int8_t *qh, const float *sh, const int32_t *counts,
                              const int32_t *offsets, const int32_t *mtile_off,
                              const int32_t *order, int64_t A, const int8_t *w_d, const float *s_d,
                              int H, int F, int E, YRows y, bool fp8, hipStream_t st, Timing tm) {
  TiledArgs a{};
  a.act = qh; a.row_scale = sh; a.counts = counts; a.offsets = offsets;
  a.mtile_off = mtile_off; a.E = E;
  a.order = order;
  a.nt = gemm2_ntiles(H); a.gn = group_n(a.nt);
  a.places = xcd_places(A, E, a.nt);
  a.w = w_d; a.wscale = s_d; a.K = F; a.F = F; a.H = H; a.y = y;
  const dim3 grid((unsigned)(8 * a.places));
  if (fp8) return launch_kernel(gemm_tiled_kernel<false, true>, grid, dim3(512), st, tm, a);
  return launch_kernel(gemm_tiled_kernel<false, false>, grid, dim3(512), st, tm, a);
}

}  // namespace moe
