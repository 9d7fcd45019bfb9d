// abi.hip -- host side of the C ABI declared in include/moe_w8a8.h:
// argument validation (before anything touches HIP), workspace carving and
// the launch sequence of one forward / calibrate call on the caller's stream.
#include <math.h>

#include <mutex>

#include "moe_internal.h"
#include "moe_w8a8.h"

namespace moe {

namespace {
constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Streaming kernels are used while experts get few rows on average; past
// that the tiled kernels reuse each weight panel across 256-row tiles.
constexpr int64_t kStreamMaxAvgRows = 32;

bool dims_valid(const moe_w8a8_dims *d) {
  return d && d->hidden > 0 && d->ffn > 0 && d->num_experts > 0 && d->top_k > 0 &&
         d->top_k <= d->num_experts;
}
bool dims_supported(const moe_w8a8_dims *d) {
  return d->hidden % 256 == 0 && d->hidden <= 65536 && d->ffn % 128 == 0 && d->ffn <= 65536 &&
         d->num_experts <= kMaxExperts && d->top_k <= kMaxTopK;
}
// The kernels index assignments and permuted rows in int32: refuse a batch
// whose T*k, or whose padded row count T*k + 15*min(T*k, E) (each expert group
// rounded up to 16 rows), reaches 2^31. T*k is bounded by a division first, so
// no product can overflow int64 for a huge T.
bool too_many_rows(int64_t T, int k, int E) {
  const int64_t lim = ((int64_t)1 << 31) - 1;
  if (T > lim / k) return true;
  const int64_t A = T * k;
  return A + 15 * (A < E ? A : (int64_t)E) > lim;
}
// More calibration tokens than any device holds: n_calib * H >= 2^61 values
// (2^62 bytes of bf16), decided without forming the product.
bool too_many_calib(int64_t n_calib, int H) { return n_calib > ((int64_t)1 << 61) / H - 1; }
// p is NULL or a multiple of a bytes.
bool al(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
// Alignment the kernels rely on (the header's rule): 16 bytes for the arrays
// they move 16 bytes at a time (tokens, weight codes, inv_smooth, the router
// matrix), 8 for the output, 4 for the other fp32/int32 arrays, 256 for a
// workspace (its regions are laid out in 256-byte steps).
bool fwd_aligned(const moe_w8a8_weights *wt, const uint16_t *x, const float *router_logits,
                 const int32_t *topk_ids, const float *topk_w, const uint16_t *out,
                 const void *workspace) {
  return al(x, 16) && al(out, 8) && al(wt->w_gate_up, 16) && al(wt->w_down, 16) &&
         al(wt->inv_smooth, 16) && al(wt->w_router, 16) && al(wt->s_gate_up, 4) &&
         al(wt->s_down, 4) && al(wt->act_clip, 4) && al(router_logits, 4) && al(topk_ids, 4) &&
         al(topk_w, 4) && al(workspace, 256);
}
}  // namespace

FwdLayout fwd_layout(int64_t T, int H, int F, int E, int k) {
  FwdLayout L{};
  const int64_t A = T * k;
  L.nblk = (T + route_tokens(T) - 1) / route_tokens(T);
  L.P = A + 15 * (A < E ? A : (int64_t)E);
  const size_t P16 = (size_t)((L.P + 15) / 16) * 16;  // rows of the tiled operands
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes); return at; };
  L.ids = take(sizeof(int32_t) * A);
  L.wts = take(sizeof(float) * A);
  // sized for the finest routing block (16 tokens), so that the workspace
  // never shrinks as T grows past a block-size step
  L.blk_hist = take(sizeof(int32_t) * (size_t)((T + 15) / 16) * E);
  L.counts = take(sizeof(int32_t) * E);
  L.offsets = take(sizeof(int32_t) * (E + 1));
  L.poffsets = take(sizeof(int32_t) * (E + 1));
  L.mtile_off = take(sizeof(int32_t) * (E + 1));
  L.tile_order = take(sizeof(int32_t) * tile_order_ints(A, E, F, H));
  L.sorted = take(sizeof(int32_t) * (size_t)L.P);
  L.row_of = take(sizeof(int32_t) * A);
  L.qx = take((size_t)T * H);
  L.sx = take(sizeof(float) * T);
  L.h = take(sizeof(float) * (size_t)L.P * F);
  L.amax = take(sizeof(uint32_t) * (size_t)L.P);
  L.qh = take(P16 * F);
  L.sh = take(sizeof(float) * (size_t)L.P);
  // y rows: fp32 (streaming path) or int16 codes + scales (tiled path) in
  // the same region, sized for the larger
  L.y = take(sizeof(float) * (size_t)L.P * H);
  L.rpart = take(sizeof(float) * (size_t)router_parts(H) * (size_t)T * (size_t)E);
  L.total = o;
  return L;
}

// 1-based rank of the nearest-rank percentile p of N values: ceil(p/100 * N)
// in fp64, clamped to [1, N].
int64_t percentile_rank(float p, int64_t N) {
  int64_t r = (int64_t)ceil((double)p / 100.0 * (double)N);
  if (r < 1) r = 1;
  if (r > N) r = N;
  return r;
}

size_t calib_ws_bytes(int H) { return align_up(sizeof(uint32_t) * H) * 2; }

}  // namespace moe

using namespace moe;

extern "C" size_t moe_w8a8_workspace_size(const moe_w8a8_dims *d, int64_t T) {
  if (!dims_valid(d) || !dims_supported(d) || T < 0) return 0;
  if (too_many_rows(T, d->top_k, d->num_experts)) return 0;
  const size_t f = fwd_layout(T, d->hidden, d->ffn, d->num_experts, d->top_k).total;
  const size_t c = calib_ws_bytes(d->hidden);
  return f > c ? f : c;
}

extern "C" const char *moe_w8a8_strerror(int code) {
  switch (code) {
    case MOE_W8A8_OK: return "success";
    case MOE_W8A8_ERR_INVALID: return "invalid argument";
    case MOE_W8A8_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_W8A8_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_W8A8_ERR_HIP: return "HIP runtime error";
    case MOE_W8A8_ERR_SCRATCH:
      return "batch too large for the static scratch of moe_w8a8_forward_noalloc";
    default: return "unknown error code";
  }
}

#define MOE_CHECK(expr)                                  \
  do {                                                   \
    if ((expr) != hipSuccess) return MOE_W8A8_ERR_HIP;   \
  } while (0)

extern "C" int moe_w8a8_pack(int64_t count, int32_t N, int32_t K, const int8_t *src, int8_t *dst,
                             void *stream) {
  if (count <= 0 || N <= 0 || K <= 0 || !src || !dst) return MOE_W8A8_ERR_INVALID;
  if ((uintptr_t)src % 16 != 0 || (uintptr_t)dst % 16 != 0) return MOE_W8A8_ERR_INVALID;
  if (N % 16 != 0 || K % 64 != 0) return MOE_W8A8_ERR_UNSUPPORTED;
  if ((int64_t)N * K > ((int64_t)1 << 40) / count) return MOE_W8A8_ERR_INVALID;
  const uintptr_t bytes = (uintptr_t)(count * (int64_t)N * K);
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return MOE_W8A8_ERR_INVALID;  // overlap
  MOE_CHECK(launch_pack(src, dst, count, N, K, (hipStream_t)stream));
  return MOE_W8A8_OK;
}

extern "C" int moe_w8a8_router_logits(const moe_w8a8_dims *d, const uint16_t *x, int64_t T,
                                      const uint16_t *w_router, float *logits, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  if (!dims_valid(d) || T < 0) return MOE_W8A8_ERR_INVALID;
  if (T == 0) return dims_supported(d) ? MOE_W8A8_OK : MOE_W8A8_ERR_UNSUPPORTED;
  if (!x || !w_router || !logits) return MOE_W8A8_ERR_INVALID;
  if (!al(x, 16) || !al(w_router, 16) || !al(logits, 4) || !al(workspace, 256))
    return MOE_W8A8_ERR_INVALID;
  if (too_many_rows(T, d->top_k, d->num_experts)) return MOE_W8A8_ERR_INVALID;
  if (!dims_supported(d)) return MOE_W8A8_ERR_UNSUPPORTED;
  const int H = d->hidden, E = d->num_experts;
  const int parts = router_parts(H);
  hipStream_t st = (hipStream_t)stream;
  if (parts == 1) {
    MOE_CHECK(launch_router_proj(x, w_router, T, E, H, logits, st, Timing{}));
    return MOE_W8A8_OK;
  }
  const FwdLayout L = fwd_layout(T, H, d->ffn, E, d->top_k);
  if (!workspace || workspace_bytes < L.total) return MOE_W8A8_ERR_WORKSPACE;
  float *rpart = (float *)((char *)workspace + L.rpart);
  MOE_CHECK(launch_router_proj(x, w_router, T, E, H, rpart, st, Timing{}));
  MOE_CHECK(launch_router_sum(rpart, parts, T, E, logits, st));
  return MOE_W8A8_OK;
}

extern "C" int moe_w8a8_calibrate_clip(const moe_w8a8_dims *d, float percentile,
                                       const uint16_t *calib_x, int64_t n_calib,
                                       const float *inv_smooth, float *act_clip, void *stream) {
  if (!dims_valid(d) || !inv_smooth || !act_clip || n_calib < 0 || (n_calib > 0 && !calib_x) ||
      !(percentile > 0.0f && percentile <= 100.0f))
    return MOE_W8A8_ERR_INVALID;
  if (!al(calib_x, 2) || !al(inv_smooth, 4) || !al(act_clip, 4)) return MOE_W8A8_ERR_INVALID;
  if (too_many_calib(n_calib, d->hidden)) return MOE_W8A8_ERR_INVALID;
  if (!dims_supported(d)) return MOE_W8A8_ERR_UNSUPPORTED;
  const int H = d->hidden;
  const int64_t N = n_calib * (int64_t)H;
  const int64_t m = N > 0 ? N - percentile_rank(percentile, N) + 1 : 1;
  MOE_CHECK(launch_calib_clip(calib_x, n_calib, H, inv_smooth, m, act_clip, (hipStream_t)stream));
  return MOE_W8A8_OK;
}

extern "C" int moe_w8a8_calibrate(const moe_w8a8_dims *d, float alpha, const uint16_t *calib_x,
                                  int64_t n_calib, const float *w_gate, const float *w_up,
                                  const float *w_down, const moe_w8a8_weights *out,
                                  void *workspace, size_t workspace_bytes, void *stream) {
  if (!dims_valid(d) || !out || !w_gate || !w_up || !w_down || n_calib < 0 ||
      (n_calib > 0 && !calib_x) || !(alpha >= 0.0f && alpha <= 1.0f))
    return MOE_W8A8_ERR_INVALID;
  if (!out->w_gate_up || !out->w_down || !out->s_gate_up || !out->s_down || !out->smooth ||
      !out->inv_smooth)
    return MOE_W8A8_ERR_INVALID;
  if (out->format != MOE_W8A8_FORMAT_INT8 && out->format != MOE_W8A8_FORMAT_FP8)
    return MOE_W8A8_ERR_INVALID;
  if (!al(calib_x, 2) || !al(w_gate, 4) || !al(w_up, 4) || !al(w_down, 4) ||
      !al(out->w_gate_up, 16) || !al(out->w_down, 16) || !al(out->s_gate_up, 4) ||
      !al(out->s_down, 4) || !al(out->smooth, 4) || !al(out->inv_smooth, 4) ||
      !al(workspace, 256))
    return MOE_W8A8_ERR_INVALID;
  if (too_many_calib(n_calib, d->hidden)) return MOE_W8A8_ERR_INVALID;
  if (!dims_supported(d)) return MOE_W8A8_ERR_UNSUPPORTED;
  const int H = d->hidden, F = d->ffn, E = d->num_experts;
  if (!workspace || workspace_bytes < calib_ws_bytes(H)) return MOE_W8A8_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  uint32_t *ax = (uint32_t *)workspace;
  uint32_t *aw = (uint32_t *)((char *)workspace + calib_ws_bytes(H) / 2);
  MOE_CHECK(launch_calib_colmax(calib_x, n_calib, w_gate, w_up, H, F, E, ax, aw, st));
  MOE_CHECK(launch_calib_smooth(ax, aw, alpha, H, out->smooth, out->inv_smooth, st));
  MOE_CHECK(launch_calib_quant(w_gate, w_up, w_down, out->smooth, H, F, E, out->w_gate_up,
                               out->s_gate_up, out->w_down, out->s_down,
                               out->format == MOE_W8A8_FORMAT_FP8, st));
  return MOE_W8A8_OK;
}

namespace {
// The forward on a given workspace (the caller's, or the static scratch).
int forward_impl(const moe_w8a8_dims *d, const moe_w8a8_weights *wt, const uint16_t *x,
                 int64_t T, const float *router_logits, const int32_t *topk_ids,
                 const float *topk_w, float capacity_factor, uint16_t *out, void *workspace,
                 size_t workspace_bytes, const moe_w8a8_debug *dbg, void *stream) {
  if (!dims_valid(d) || !wt || T < 0) return MOE_W8A8_ERR_INVALID;
  if (T == 0) return dims_supported(d) ? MOE_W8A8_OK : MOE_W8A8_ERR_UNSUPPORTED;
  const bool routed = router_logits != nullptr;
  const bool pre = topk_ids != nullptr || topk_w != nullptr;
  const bool project = !routed && !pre;
  if ((routed && pre) || (pre && (!topk_ids || !topk_w)) || (project && !wt->w_router))
    return MOE_W8A8_ERR_INVALID;
  if (too_many_rows(T, d->top_k, d->num_experts)) return MOE_W8A8_ERR_INVALID;
  if (!x || !out || !wt->w_gate_up || !wt->w_down || !wt->s_gate_up || !wt->s_down ||
      !wt->inv_smooth)
    return MOE_W8A8_ERR_INVALID;
  if (!fwd_aligned(wt, x, router_logits, topk_ids, topk_w, out, workspace))
    return MOE_W8A8_ERR_INVALID;
  if (isnan(capacity_factor)) return MOE_W8A8_ERR_INVALID;
  const float sat_p = wt->act_sat_percentile;
  if (!(sat_p == 0.0f || (sat_p > 0.0f && sat_p <= 100.0f))) return MOE_W8A8_ERR_INVALID;
  if (wt->format != MOE_W8A8_FORMAT_INT8 && wt->format != MOE_W8A8_FORMAT_FP8)
    return MOE_W8A8_ERR_INVALID;
  const bool fp8 = wt->format == MOE_W8A8_FORMAT_FP8;
  if (dbg && (dbg->gemm_path < 0 || dbg->gemm_path > 2)) return MOE_W8A8_ERR_INVALID;
  // the streaming GEMM1 writes the debug accumulators 16 bytes at a time
  if (dbg && (!al(dbg->acc1, 16) || !al(dbg->topk_ids, 4) || !al(dbg->topk_w, 4) ||
              !al(dbg->expert_counts, 4) || !al(dbg->expert_offsets, 4) ||
              !al(dbg->sorted_assign, 4) || !al(dbg->row_of, 4) || !al(dbg->sx, 4) ||
              !al(dbg->h, 4) || !al(dbg->sh, 4) || !al(dbg->y, 4) || !al(dbg->router_logits, 4)))
    return MOE_W8A8_ERR_INVALID;
  if (!dims_supported(d)) return MOE_W8A8_ERR_UNSUPPORTED;
  const int H = d->hidden, F = d->ffn, E = d->num_experts, k = d->top_k;
  ActClip ac{wt->act_clip, 0};
  if (sat_p > 0.0f) {
    ac.sat_m = (int)(H - percentile_rank(sat_p, H) + 1);
    if (ac.sat_m > kMaxSatM) return MOE_W8A8_ERR_UNSUPPORTED;
  }
  const FwdLayout L = fwd_layout(T, H, F, E, k);
  if (!workspace || workspace_bytes < L.total) return MOE_W8A8_ERR_WORKSPACE;

  const int64_t A = T * k;
  int64_t capacity = 0;
  if (capacity_factor > 0.0f) {
    const double c = ceil((double)capacity_factor * (double)T * (double)k / (double)E);
    capacity = c >= (double)A ? A : (int64_t)c;
    if (capacity < 1) capacity = 1;
  }
  int path = dbg ? dbg->gemm_path : 0;
  if (path == 0) path = A <= kStreamMaxAvgRows * E ? 1 : 2;

  char *ws = (char *)workspace;
  int32_t *ids = (int32_t *)(ws + L.ids);
  float *wts = (float *)(ws + L.wts);
  int32_t *blk_hist = (int32_t *)(ws + L.blk_hist);
  int32_t *counts = (int32_t *)(ws + L.counts);
  int32_t *offsets = (int32_t *)(ws + L.offsets);
  int32_t *poffsets = (int32_t *)(ws + L.poffsets);
  int32_t *mtile_off = (int32_t *)(ws + L.mtile_off);
  int32_t *tile_order = (int32_t *)(ws + L.tile_order);
  int32_t *sorted = (int32_t *)(ws + L.sorted);
  int32_t *row_of = (int32_t *)(ws + L.row_of);
  int8_t *qx = (int8_t *)(ws + L.qx);
  float *sx = (float *)(ws + L.sx);
  float *h = (float *)(ws + L.h);
  uint32_t *amax = (uint32_t *)(ws + L.amax);
  int8_t *qh = (int8_t *)(ws + L.qh);
  float *sh = (float *)(ws + L.sh);
  // y rows: the tiled path codes them to int16 with a scale per 16 columns
  // (the codes first, then the scales, inside the fp32-sized region)
  YRows y{(float *)(ws + L.y), nullptr, nullptr};
  if (path == 2) {
    const size_t codes = (size_t)L.P * H * sizeof(int16_t);
    y = YRows{nullptr, (int16_t *)(ws + L.y), (float *)(ws + L.y + (codes + 255) / 256 * 256)};
  }
  int32_t *acc1_dbg = dbg ? dbg->acc1 : nullptr;
  hipStream_t st = (hipStream_t)stream;

  const bool small = A <= kSmallA;

  // Stage events: pair s is stamped by the dispatch of the launch that
  // performs stage s; a launch that fuses several stages takes the pair of
  // the first of them, and a stage of two launches is timed from the start
  // of the first to the end of the second.
  void **ev = dbg ? dbg->stage_events : nullptr;
  auto tm = [&](int s, bool start = true, bool stop = true) -> Timing {
    Timing t;
    if (ev) {
      if (start) t.start = (hipEvent_t)ev[2 * s];
      if (stop) t.stop = (hipEvent_t)ev[2 * s + 1];
    }
    return t;
  };
  enum { kRoute, kScan, kScatter, kActQ, kG1, kReq, kG2, kComb, kRouter };

  LogitPlanes lp{router_logits, 1, 0};
  if (project) {
    float *rpart = (float *)(ws + L.rpart);
    MOE_CHECK(launch_router_proj(x, wt->w_router, T, E, H, rpart, st, tm(kRouter)));
    lp = LogitPlanes{rpart, router_parts(H), T * (int64_t)E};
  }

  // The tiled path's tile orders are built by extra blocks of the scatter
  // launch (a small batch's fused prologue has no such launch: its tiles run
  // in expert-major order).
  const TileOrderArgs to = tile_order_args(A, E, F, H, counts, mtile_off,
                                           path == 2 && !small ? tile_order : nullptr);
  if (small) {
    MOE_CHECK(launch_prologue_small(lp, topk_ids, topk_w, (int)T, E, k, capacity, ids,
                                    wts, counts, offsets, poffsets, mtile_off, sorted, row_of,
                                    (int)L.P, x, wt->inv_smooth, H, qx, sx, amax, ac, fp8, st,
                                    tm(kRoute)));
  } else {
    MOE_CHECK(launch_route_hist(lp, topk_ids, topk_w, T, E, k, ids, wts, blk_hist,
                                amax, sorted, L.P, st, tm(kRoute)));
    MOE_CHECK(launch_scan(blk_hist, L.nblk, E, capacity, counts, offsets, poffsets, mtile_off, st,
                          tm(kScan)));
    MOE_CHECK(launch_scatter(ids, blk_hist, poffsets, T, E, k, capacity, sorted, row_of, to, st,
                             tm(kScatter)));
  }
  const int32_t *order1 = to.order[0], *order2 = to.order[1];
  if (path == 1) {
    if (!small)
      MOE_CHECK(launch_act_quant(x, wt->inv_smooth, T, H, qx, sx, ac, fp8, st, tm(kActQ)));
    MOE_CHECK(launch_gemm1_stream(qx, sx, sorted, k, counts, poffsets, offsets, wt->w_gate_up,
                                  wt->s_gate_up, H, F, E, h, amax, acc1_dbg, fp8, st, tm(kG1)));
  } else {
    // GEMM1 gathers its activation rows from qx as it loads them.
    if (!small)
      MOE_CHECK(launch_act_quant(x, wt->inv_smooth, T, H, qx, sx, ac, fp8, st, tm(kActQ)));
    MOE_CHECK(launch_gemm1_tiled(qx, sx, sorted, k, counts, poffsets, offsets, mtile_off, order1,
                                 A, wt->w_gate_up, wt->s_gate_up, H, F, E, h, amax, acc1_dbg, fp8,
                                 st, tm(kG1)));
  }
  MOE_CHECK(launch_requant(h, amax, poffsets, E, L.P, F, qh, sh, fp8, st, tm(kReq)));
  if (path == 1)
    MOE_CHECK(launch_gemm2_stream(qh, sh, counts, poffsets, wt->w_down, wt->s_down, H, F, E, y.f,
                                  fp8, st, tm(kG2)));
  else
    MOE_CHECK(launch_gemm2_tiled(qh, sh, counts, poffsets, mtile_off, order2, A, wt->w_down,
                                 wt->s_down, H, F, E, y, fp8, st, tm(kG2)));
  MOE_CHECK(launch_combine(y, wts, row_of, T, H, k, out, st, tm(kComb)));

  if (dbg) {
    auto cp = [&](void *dst, const void *src, size_t bytes) -> hipError_t {
      if (!dst || bytes == 0) return hipSuccess;
      return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st);
    };
    MOE_CHECK(cp(dbg->topk_ids, ids, sizeof(int32_t) * A));
    MOE_CHECK(cp(dbg->topk_w, wts, sizeof(float) * A));
    MOE_CHECK(cp(dbg->expert_counts, counts, sizeof(int32_t) * E));
    MOE_CHECK(cp(dbg->expert_offsets, offsets, sizeof(int32_t) * (E + 1)));
    MOE_CHECK(cp(dbg->qx, qx, (size_t)T * H));
    MOE_CHECK(cp(dbg->sx, sx, sizeof(float) * T));
    if (dbg->router_logits) {
      if (project)
        MOE_CHECK(launch_router_sum(lp.p, lp.nparts, T, E, dbg->router_logits, st));
      else if (routed)
        MOE_CHECK(cp(dbg->router_logits, router_logits, sizeof(float) * T * E));
    }
    if (dbg->sorted_assign || dbg->h || dbg->qh || dbg->sh || dbg->y)
      MOE_CHECK(launch_debug_rows(offsets, poffsets, E, A, sorted, h, qh, sh, y, F, H,
                                  dbg->sorted_assign, dbg->h, dbg->qh, dbg->sh, dbg->y, st));
    if (dbg->row_of)
      MOE_CHECK(launch_debug_row_of(row_of, ids, offsets, poffsets, A, dbg->row_of, st));
  }
  return MOE_W8A8_OK;
}
}  // namespace

extern "C" int moe_w8a8_forward(const moe_w8a8_dims *d, const moe_w8a8_weights *wt,
                                const uint16_t *x, int64_t T, const float *router_logits,
                                const int32_t *topk_ids, const float *topk_w,
                                float capacity_factor, uint16_t *out, void *workspace,
                                size_t workspace_bytes, const moe_w8a8_debug *dbg,
                                void *stream) {
  return forward_impl(d, wt, x, T, router_logits, topk_ids, topk_w, capacity_factor, out,
                      workspace, workspace_bytes, dbg, stream);
}

// ------------------------------------------------- forward without allocation
// The workspace of moe_w8a8_forward_noalloc: a file-scope device array, one
// copy per GPU, alive until the process ends. In host code `scratch` names a
// host-side stand-in, not the device memory: its device address is taken
// once per device with hipGetSymbolAddress and only that address is used.
namespace {
static __device__ __align__(256) char scratch[MOE_W8A8_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch (resolved on the first call on it).
hipError_t scratch_on_current_device(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" int moe_w8a8_forward_noalloc(const moe_w8a8_dims *d, const moe_w8a8_weights *wt,
                                        const uint16_t *x, int64_t T, const float *router_logits,
                                        const int32_t *topk_ids, const float *topk_w,
                                        float capacity_factor, uint16_t *out,
                                        const moe_w8a8_debug *dbg, void *stream) {
  if (!dims_valid(d) || !wt || T < 0) return MOE_W8A8_ERR_INVALID;
  if (T == 0) return dims_supported(d) ? MOE_W8A8_OK : MOE_W8A8_ERR_UNSUPPORTED;
  if (too_many_rows(T, d->top_k, d->num_experts)) return MOE_W8A8_ERR_INVALID;
  if (!dims_supported(d)) return MOE_W8A8_ERR_UNSUPPORTED;
  if (moe_w8a8_workspace_size(d, T) > MOE_W8A8_SCRATCH_BYTES) return MOE_W8A8_ERR_SCRATCH;
  if (!fwd_aligned(wt, x, router_logits, topk_ids, topk_w, out, nullptr))
    return MOE_W8A8_ERR_INVALID;
  void *ws = nullptr;
  MOE_CHECK(scratch_on_current_device(&ws));
  return forward_impl(d, wt, x, T, router_logits, topk_ids, topk_w, capacity_factor, out, ws,
                      MOE_W8A8_SCRATCH_BYTES, dbg, stream);
}
