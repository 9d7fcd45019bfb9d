// moe_internal.h -- internal declarations shared by the HIP sources of
// libmoe_w8a8 (kernel launchers, device helpers, workspace carving).
// Not part of the public ABI (include/moe_w8a8.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Tokens routed (and histogrammed) per block of the routing kernels for a
// batch of T tokens: the fewest of 64, 32, 16 per block that still give at
// most 256 blocks, so that a few thousand tokens spread over the whole chip
// (one token per wavefront) while large batches keep the per-block
// histograms that the scan reads few.
inline int route_tokens(int64_t T) { return T <= 4096 ? 16 : (T <= 8192 ? 32 : 64); }
// Rows per M tile of the tiled grouped GEMMs.
constexpr int kTiledBM = 256;
// A tiled GEMM with at most this many tiles (three rounds of the 256
// compute units) gets a tile order: ranges of equal estimated time per XCD,
// each run longest first. Its grid then gives each XCD at least
// kTileOrderPlaces places (a range holds at most ~0.22 of the tiles).
constexpr int kTileOrderMaxTiles = 3 * 256;
constexpr int kTileOrderPlaces = 192;
// What the blocks that build the tile orders need: per GEMM g, its N tiles
// per expert nt[g], N tiles per group gn[g], the places per XCD of its grid
// cap[g] and its region order[g] (NULL: none built).
struct TileOrderArgs {
  const int32_t *counts, *mtile_off;
  int E;
  int nt[2], gn[2], cap[2];
  int32_t *order[2];
};
// Maximum experts (LDS histograms are sized for it).
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
// Up to this many assignments (T*k) the routing, grouping and activation
// quantisation run as one fused launch (one block does the grouping).
constexpr int kSmallA = 2048;
// Hidden channels per part of the router projection's fixed summation order.
constexpr int kRouterPart = 512;

// Clip of the per-token activation quantiser: the row is quantised at a
// level below its maximum when *clip is a positive static threshold, or when
// sat_m > 1 (dynamic saturation: at most the row's sat_m-th largest |v|).
// Zero thresholds leave the level alone.
constexpr int kMaxSatM = 16;  // largest supported sat_m
struct ActClip {
  const float *clip;  // device fp32 [1], or NULL
  int sat_m;          // 0 or 1: off
};

// GEMM2's output rows y as the combine reads them, in one of two forms:
//  - f != NULL: fp32 rows [rows][H] (the streaming path: a decode step's y is
//    small, and its GEMM2 writes each row's values as they come);
//  - f == NULL: y[row][n] held as the int16 code q[row][n] times the fp32
//    scale s[row][n/16], one scale per 16 columns (the group's largest |y| /
//    32767; codes v/max as signed normalised 16-bit values), written by the
//    tiled path, whose y is T*k rows: 2.25 bytes per value through HBM
//    instead of 4. The rounding error is at most about 2^-16 of the group's
//    largest value, far below what the output's parity bound allows.
constexpr int kYGroup = 16;
constexpr float kYCodeMax = 32767.0f;
struct YRows {
  float *f;    // [rows][H] fp32, or NULL
  int16_t *q;  // [rows][H] codes (when f is NULL)
  float *s;    // [rows][H / 16] scales (when f is NULL)
};

// Router logits as the routing kernels read them: the logit of (t, e) is
// the sum, in order s = 0..nparts-1, of p[s * stride + t * E + e] (one plane
// when the caller gives the logits, one per part of the router projection).
struct LogitPlanes {
  const float *p;  // NULL: pre-routed
  int nparts;
  int64_t stride;
};

// ------------------------------------------------------------ device helpers
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
// fp32 -> bf16, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// Symmetric INT8 code of v for reciprocal scale rr = fl32(127/amax):
// rint(fl32(v*rr)) clamped to [-127, 127].
__device__ __forceinline__ int q8(float v, float rr) {
  float c = __builtin_rintf(v * rr);
  c = __builtin_fminf(__builtin_fmaxf(c, -127.0f), 127.0f);
  return (int)c;
}
// Code format of the expert path ("超大规模模型推理的Day0适配实践" §二.1:
// expert layers in INT8 or FP8; §四: activations follow the weights' format).
// kFp8Max is the largest finite OCP e4m3 value, the level a range maps to.
constexpr float kFp8Max = 448.0f;
// Four FP8 (OCP e4m3) codes of fl32(v*rr), packed little-endian: each
// product is clamped to [-448, 448] first (the conversion itself does not
// saturate), then rounded to nearest, ties to even, by the hardware
// conversion (the sign of zero is kept).
__device__ __forceinline__ uint32_t f8x4(float a, float b, float c, float d, float rr) {
  auto cl = [&](float v) { return __builtin_fminf(__builtin_fmaxf(v * rr, -kFp8Max), kFp8Max); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
  return (uint32_t)w;
}
// Four codes of v*rr in the given format (INT8: q8; FP8: f8x4).
__device__ __forceinline__ uint32_t codes4(const float *v, float rr, bool fp8) {
  if (fp8) return f8x4(v[0], v[1], v[2], v[3], rr);
  return (uint32_t)(q8(v[0], rr) & 0xff) | ((uint32_t)(q8(v[1], rr) & 0xff) << 8) |
         ((uint32_t)(q8(v[2], rr) & 0xff) << 16) | ((uint32_t)(q8(v[3], rr) & 0xff) << 24);
}
// y codes: v / gm as signed normalised 16-bit values (v_cvt_pknorm_i16_f32:
// clamp to [-1, 1], times 32767, rounded), two per 32-bit word, for a group
// whose largest |y| is gm; the group's scale is gm / 32767. Groups whose
// largest value is below 1e-30 get codes 0 and scale 0.
__device__ __forceinline__ float y16_inv(float gm) { return gm > 1e-30f ? 1.0f / gm : 0.0f; }
__device__ __forceinline__ int y16x2(float a, float b, float inv) {
  return __builtin_bit_cast(int, __builtin_amdgcn_cvt_pknorm_i16(a * inv, b * inv));
}
__device__ __forceinline__ float y16_scale(float gm) {
  return gm > 1e-30f ? gm / kYCodeMax : 0.0f;
}
// Byte offset of the 1 KB fragment tile (n_tile, k_tile) of a fragment-tiled
// [N][K] INT8 matrix.
__device__ __forceinline__ size_t frag_tile(int n_tile, int k_tile, int K) {
  return ((size_t)n_tile * (size_t)(K >> 6) + (size_t)k_tile) << 10;
}
// Maximum over the wavefront of a non-negative value (a |x| maximum), in
// every lane. Non-negative floats order as their bit patterns. DPP moves
// instead of LDS permutes: row_shr 1, 2, 4, 8 leave each 16-lane row's
// maximum in its lane 15; row_bcast 15 into rows 1 and 3 and row_bcast 31
// into rows 2 and 3 gather all four in lane 63, which is then read out.
__device__ __forceinline__ float wave_max(float v) {
  auto step = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
  uint32_t m = __float_as_uint(v);
  m = step(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x111, 0xF, 0xF, false));
  m = step(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x112, 0xF, 0xF, false));
  m = step(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x114, 0xF, 0xF, false));
  m = step(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x118, 0xF, 0xF, false));
  m = step(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x142, 0xA, 0xF, false));
  m = step(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x143, 0xC, 0xF, false));
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)m, 63));
}
// Inclusive prefix sum over the wavefront (every lane active), by the same
// DPP steps: within each 16-lane row, lanes add the partial sums 1, 2, 4 and
// 8 lanes below them (lanes with no such source add the 0 they are given);
// then rows 1 and 3 add the total of the row below, and rows 2 and 3 the
// total of rows 0 and 1.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}
// Sum over the wavefront, in every lane.
__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}
// One DPP move of a 64-bit value (both halves from the same source lane;
// lanes without a source get 0).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, kCtrl, kRowMask, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), kCtrl, kRowMask, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
// Inclusive prefix sum of 64-bit values over the wavefront (every lane active).
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  v += dpp_u64<0x111, 0xF>(v);
  v += dpp_u64<0x112, 0xF>(v);
  v += dpp_u64<0x114, 0xF>(v);
  v += dpp_u64<0x118, 0xF>(v);
  v += dpp_u64<0x142, 0xA>(v);
  v += dpp_u64<0x143, 0xC>(v);
  return v;
}
// Maximum of 64-bit unsigned values over the wavefront, in every lane (every
// lane active; 0 is the identity).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  v = mx(v, dpp_u64<0x111, 0xF>(v));
  v = mx(v, dpp_u64<0x112, 0xF>(v));
  v = mx(v, dpp_u64<0x114, 0xF>(v));
  v = mx(v, dpp_u64<0x118, 0xF>(v));
  v = mx(v, dpp_u64<0x142, 0xA>(v));
  v = mx(v, dpp_u64<0x143, 0xC>(v));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ v4i mfma16(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16i mfma32(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
// FP8 (e4m3) x FP8 -> fp32 with unit block scales (E8M0 127 = 1.0). The
// 32 bytes a lane gives per operand are two 16-byte k-chunks, a0|a1 and
// b0|b1: the instruction pairs A and B bytes by the same lane position, so
// chunks taken alike from both operands (the same INT8-layout k-chunks)
// make the full dot product, whatever k order the hardware assigns.
__device__ __forceinline__ v8i cat8(v4i x, v4i y) {
  return v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}
__device__ __forceinline__ v4f mfma16f8(v4i a0, v4i a1, v4i b0, v4i b1, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cat8(a0, a1), cat8(b0, b1), c, 0, 0, 0,
                                                          127, 0, 127);
}
__device__ __forceinline__ v16f mfma32f8(v4i a0, v4i a1, v4i b0, v4i b1, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat8(a0, a1), cat8(b0, b1), c, 0, 0, 0,
                                                         127, 0, 127);
}
#endif

// ------------------------------------------------------------------ launches
// Optional timing of one launch: the events are stamped by the kernel's own
// dispatch (hipExtLaunchKernel: start and end of its execution), so timing a
// stage adds no marker packet, and no gap, between the layer's kernels.
struct Timing {
  hipEvent_t start = nullptr, stop = nullptr;
};
// The launch's own error: hipGetLastError also returns an error that an
// earlier call in the process (another library's included) left behind, so
// that one is cleared first.
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                                Timing tm, Args... args) {
  (void)hipGetLastError();
  if (tm.start || tm.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, tm.start, tm.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  return hipGetLastError();
}

// ---------------------------------------------------------------- workspace
// Regions of the forward workspace (byte offsets from its base).
// Permuted rows inside the layer are "padded": every expert's group starts on
// a 16-row boundary, so P <= A + 15*min(E, A) rows for A = T*k assignments.
struct FwdLayout {
  size_t ids, wts, blk_hist, counts, offsets, poffsets, mtile_off, tile_order, sorted, row_of,
      qx, sx, h, amax, qh, sh, y, rpart, total;
  int64_t nblk;  // routing blocks
  int64_t P;     // padded permuted rows (upper bound)
};
FwdLayout fwd_layout(int64_t T, int H, int F, int E, int k);
// Calibrate workspace: ax[H], aw[H] as uint32 float bits.
size_t calib_ws_bytes(int H);

// ----------------------------------------------------------------- launchers
// Each returns hipGetLastError() after enqueueing on `st` (timed by `tm`).
// Rows of sorted/h/amax/qh/sh/y are padded rows; offsets are dense group
// starts, poffsets the padded ones; qh is fragment-tiled.
// Fused small-batch prologue: route (or copy pre-routed ids), group, clear
// the per-row max and sorted[] over P rows, and quantise the activations.
hipError_t launch_prologue_small(LogitPlanes logits, const int32_t *ids_in, const float *w_in,
                                 int T, int E, int k, int64_t capacity, int32_t *ids, float *wts,
                                 int32_t *counts, int32_t *offsets, int32_t *poffsets,
                                 int32_t *mtile_off, int32_t *sorted, int32_t *row_of, int P,
                                 const uint16_t *x, const float *inv_s, int H, int8_t *qx,
                                 float *sx, uint32_t *amax, ActClip ac, bool fp8,
                                 hipStream_t st, Timing tm);
hipError_t launch_route_hist(LogitPlanes logits, const int32_t *ids_in, const float *w_in,
                             int64_t T, int E, int k, int32_t *ids, float *wts,
                             int32_t *blk_hist, uint32_t *amax, int32_t *sorted, int64_t P,
                             hipStream_t st, Timing tm);
int router_parts(int H);
hipError_t launch_router_proj(const uint16_t *x, const uint16_t *w_router, int64_t T, int E,
                              int H, float *part, hipStream_t st, Timing tm);
hipError_t launch_router_sum(const float *part, int nparts, int64_t T, int E, float *logits,
                             hipStream_t st);
hipError_t launch_scan(int32_t *blk_hist, int64_t nblk, int E, int64_t capacity, int32_t *counts,
                       int32_t *offsets, int32_t *poffsets, int32_t *mtile_off, hipStream_t st,
                       Timing tm);
// (with to.order[g] set, 8 more blocks per GEMM g build its tile order)
hipError_t launch_scatter(const int32_t *ids, const int32_t *blk_hist, const int32_t *poffsets,
                          int64_t T, int E, int k, int64_t capacity, int32_t *sorted,
                          int32_t *row_of, const TileOrderArgs &to, hipStream_t st, Timing tm);
hipError_t launch_act_quant(const uint16_t *x, const float *inv_s, int64_t T, int H, int8_t *qx,
                            float *sx, ActClip ac, bool fp8, hipStream_t st, Timing tm);
hipError_t launch_requant(const float *h, const uint32_t *amax, const int32_t *poffsets, int E,
                          int64_t P, int F, int8_t *qh, float *sh, bool fp8, hipStream_t st,
                          Timing tm);
hipError_t launch_gemm1_stream(const int8_t *qx, const float *sx, const int32_t *sorted, int k,
                               const int32_t *counts, const int32_t *poffsets,
                               const int32_t *dense_off, const int8_t *w_gu, const float *s_gu,
                               int H, int F, int E, float *h, uint32_t *amax, int32_t *acc1_dbg,
                               bool fp8, hipStream_t st, Timing tm);
hipError_t launch_gemm2_stream(const int8_t *qh, const float *sh, const int32_t *counts,
                               const int32_t *poffsets, const int8_t *w_d, const float *s_d, int H,
                               int F, int E, float *y, bool fp8, hipStream_t st, Timing tm);
// Tile orders of the two tiled GEMMs (gemm_tiled.hip, tile_order_block in
// layer_device.h): each GEMM's region is a flag, the tile count of each XCD
// and its tiles; with the flag 0 (or no region) a GEMM runs its tiles in
// expert-major order. The regions are written by extra blocks of the
// scatter launch. tile_order_ints: both regions' size for A assignments.
size_t tile_order_ints(int64_t A, int E, int F, int H);
TileOrderArgs tile_order_args(int64_t A, int E, int F, int H, const int32_t *counts,
                              const int32_t *mtile_off, int32_t *region);
hipError_t launch_gemm1_tiled(const int8_t *qx, const float *sx, const int32_t *sorted, int k,
                              const int32_t *counts, const int32_t *offsets,
                              const int32_t *dense_off, const int32_t *mtile_off,
                              const int32_t *order, int64_t A, const int8_t *w_gu,
                              const float *s_gu, int H, int F, int E, float *h, uint32_t *amax,
                              int32_t *acc1_dbg, bool fp8, hipStream_t st, Timing tm);
hipError_t launch_gemm2_tiled(const int8_t *qh, const float *sh, const int32_t *counts,
                              const int32_t *offsets, const int32_t *mtile_off,
                              const int32_t *order, int64_t A, const int8_t *w_d, const float *s_d,
                              int H, int F, int E, YRows y, bool fp8, hipStream_t st, Timing tm);
hipError_t launch_combine(YRows y, const float *wts, const int32_t *row_of, int64_t T,
                          int H, int k, uint16_t *out, hipStream_t st, Timing tm);
// stage outputs in dense rows (debug only)
hipError_t launch_debug_rows(const int32_t *offsets, const int32_t *poffsets, int E, int64_t A,
                             const int32_t *sorted_p, const float *h_p, const int8_t *qh_t,
                             const float *sh_p, YRows y_p, int F, int H, int32_t *sorted,
                             float *h, int8_t *qh, float *sh, float *y, hipStream_t st);
hipError_t launch_debug_row_of(const int32_t *row_of_p, const int32_t *ids, const int32_t *offsets,
                               const int32_t *poffsets, int64_t A, int32_t *row_of,
                               hipStream_t st);
// row-major [count][N][K] codes -> fragment-tiled (N % 16 == 0, K % 64 == 0)
hipError_t launch_pack(const int8_t *src, int8_t *dst, int64_t count, int N, int K,
                       hipStream_t st);
// calibrate
hipError_t launch_calib_colmax(const uint16_t *calib_x, int64_t n_calib, const float *w_gate,
                               const float *w_up, int H, int F, int E, uint32_t *ax, uint32_t *aw,
                               hipStream_t st);
hipError_t launch_calib_clip(const uint16_t *calib_x, int64_t n_calib, int H, const float *inv_s,
                             int64_t m, float *out, hipStream_t st);
hipError_t launch_calib_smooth(const uint32_t *ax, const uint32_t *aw, float alpha, int H,
                               float *s, float *inv_s, hipStream_t st);
hipError_t launch_calib_quant(const float *w_gate, const float *w_up, const float *w_down,
                              const float *s, int H, int F, int E, int8_t *w_gu, float *s_gu,
                              int8_t *w_d, float *s_d, bool fp8, hipStream_t st);

}  // namespace moe
