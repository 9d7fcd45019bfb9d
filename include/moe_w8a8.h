/*
 * moe_w8a8.h -- C ABI of the W8A8-quantised Mixture-of-Experts expert layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (one call to moe_w8a8_forward) computes, for T tokens x[T][H]:
 *   1. route    top-k experts per token from router logits (given, or
 *               projected from x by the bf16 router matrix in the same call),
 *               ties to the lower expert index, softmax weights renormalised
 *               over the chosen k
 *               ("超大规模模型推理的Day0适配实践" §四: the fused MoE operator's
 *               top-k must equal the reference, tie-break included);
 *   2. permute  group the T*k (token, slot) assignments expert by expert,
 *               (token, slot) order inside a group, an optional expert
 *               capacity dropping the overflow (same page, §二.2);
 *   3. quantise each token to INT8 per token after dividing by the
 *               SmoothQuant scales ("MiniMax-M3 W8A8 inference on K100AI",
 *               mhpq.cn/news/1068415, §3.2 and §6.4), at the token's absolute
 *               maximum or, when a clip is set, at the smaller of that and
 *               the clip thresholds (values beyond saturate at +-127: K100AI
 *               page §6.4; "一晚上完成MoE模型推理优化…" §3.2);
 *   4. GEMM1    per expert, INT8 x INT8 -> INT32 gate and up projections,
 *               dequantised per token and per output channel, h = silu(g)*u,
 *               requantised to INT8 per (token, expert) row (K100AI page
 *               §1.2 and §4.3: INT8 GEMM with integer accumulation; stay in
 *               the INT8 domain between consecutive matmuls);
 *   5. GEMM2    per expert, INT8 down projection, dequantised per row and
 *               per output channel to fp32 (for large batches held until the
 *               combine as int16 codes with one fp32 scale per 16 outputs,
 *               error at most ~2^-16 of the group's largest value);
 *   6. combine  out[t] = sum over kept slots of w[t][j] * y[row], summed in
 *               fp32 and rounded to bfloat16 (Day0 page §四: un-sort and
 *               weighted sum).
 * moe_w8a8_calibrate prepares the quantised weights (K100AI page §3.2:
 * SmoothQuant with migration strength alpha, per-output-channel weights).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent) owned
 *    by the caller; nothing is allocated or freed inside the library and no
 *    library state survives a call. Layouts are row-major unless stated.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously; the library never synchronises. Calls on
 *    different streams with disjoint buffers may run concurrently.
 *  - Arguments are validated on the host before anything is enqueued; an
 *    invalid call enqueues nothing and returns a negative code. Faults inside
 *    kernels surface at the caller's next synchronisation.
 *  - bfloat16 values are passed as uint16_t bit patterns.
 */
#ifndef MOE_W8A8_H
#define MOE_W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MOE_W8A8_OK 0
#define MOE_W8A8_ERR_INVALID (-1)     /* NULL required pointer, bad size, k > E, ... */
#define MOE_W8A8_ERR_UNSUPPORTED (-2) /* shape outside the supported set (below)     */
#define MOE_W8A8_ERR_WORKSPACE (-3)   /* workspace NULL or smaller than required     */
#define MOE_W8A8_ERR_HIP (-4)         /* a HIP launch or copy reported an error      */
#define MOE_W8A8_ERR_SCRATCH (-5)     /* batch too large for the static scratch      */

/* Alignment of the device pointers every entry point takes (a violation is
 * MOE_W8A8_ERR_INVALID, before anything is enqueued): 16 bytes for arrays the
 * kernels move 16 bytes at a time (the tokens x, the packed weight codes
 * w_gate_up and w_down, inv_smooth when the forward reads it, the router
 * matrix, pack's src and dst, the debug accumulators acc1), 8 bytes for the
 * forward's output, the natural alignment of the element type for every other
 * array, and 256 bytes for a workspace (its regions are laid out in 256-byte
 * steps). hipMalloc and torch allocations satisfy all of them. */

/* Layer dimensions. Supported set: hidden H a multiple of 256 in [256, 65536];
 * ffn F a multiple of 128 in [128, 65536]; 1 <= num_experts E <= 1024;
 * 1 <= top_k k <= min(E, 32). */
typedef struct {
  int32_t hidden;      /* H */
  int32_t ffn;         /* F, the expert FFN width (SwiGLU gate/up/down) */
  int32_t num_experts; /* E, experts held on this device */
  int32_t top_k;       /* k, assignments per token */
} moe_w8a8_dims;

/* Code format of the expert path ("超大规模模型推理的Day0适配实践" §二.1: expert
 * layers in INT8 or FP8; §四: the activations take the weights' format).
 *   INT8: symmetric codes in [-127, 127], scale = range/127, integer
 *         accumulation.
 *   FP8:  OCP e4m3 codes (bias 7, 3 mantissa bits, subnormals, largest
 *         finite 448, NaN 0x7f/0xff), scale = range/448; a value is coded as
 *         the nearest e4m3 (ties to even, sign of zero kept) of
 *         clamp(fl32(v * fl32(448/range)), -448, 448); fp32 accumulation of
 *         the exact code products. */
#define MOE_W8A8_FORMAT_INT8 0
#define MOE_W8A8_FORMAT_FP8 1

/* Quantised layer weights (device memory, written by moe_w8a8_calibrate).
 *
 * Fragment-tiled INT8 layout. A weight matrix W[N][K] (N output channels,
 * K input channels; N % 16 == 0, K % 64 == 0) is stored as 1024-byte tiles of
 * 16 output channels x 64 input channels, tile (n/16, k/64) at byte offset
 *     ((n/16) * (K/64) + k/64) * 1024,
 * and inside a tile the element (n, k) at byte
 *     (((k % 64) / 16) * 16 + n % 16) * 16 + k % 16.
 * One tile is exactly one wavefront's 16-byte-per-lane load in the lane order
 * of the gfx950 INT8 matrix instructions, so weight panels stream from HBM as
 * contiguous 1 KB blocks.
 *   w_gate_up : E matrices of [2F][H], consecutive; rows 0..F-1 are the gate
 *               projection, rows F..2F-1 the up projection (smoothed).
 *   w_down    : E matrices of [H][F], consecutive (not smoothed).
 *   s_gate_up : fp32 [E][2F]  dequantisation scale per output channel.
 *   s_down    : fp32 [E][H]   dequantisation scale per output channel.
 *   smooth    : fp32 [H]      SmoothQuant scale s_j.
 *   inv_smooth: fp32 [H]      1/s_j rounded to fp32 (what forward multiplies by).
 *   w_router  : bf16 [E][H]   router projection, row e for expert e, or NULL.
 *               Not quantised ("MiniMax-M3 W8A8 inference on K100AI" §6.1:
 *               the layers at the routing stay in 16-bit floating point) and
 *               not written by moe_w8a8_calibrate.
 *   act_clip  : fp32 [1]      static activation clipping threshold c written by
 *               moe_w8a8_calibrate_clip, or NULL (no static clip). A value
 *               <= 0 also means no clip.
 *   act_sat_percentile  (a value, not a buffer) dynamic saturation of the
 *               activations: 0 = off, else p in (0, 100]: each token is
 *               quantised at most at the nearest-rank p-th percentile of its
 *               own |x_j / s_j| (the m-th largest, m = H - ceil(p/100*H) + 1,
 *               m <= 16 supported).
 *   format    : MOE_W8A8_FORMAT_INT8 or _FP8, set by the caller before
 *               moe_w8a8_calibrate (which codes the weights in it); forward
 *               codes the activations and runs the GEMMs in the same format.
 * Code of W'[n][k] is q with W' ~= q * scale[n] (INT8: codes lie in
 * [-127, 127]; FP8: W' ~= e4m3 value of q * scale[n]). */
typedef struct {
  int8_t *w_gate_up;
  int8_t *w_down;
  float *s_gate_up;
  float *s_down;
  float *smooth;
  float *inv_smooth;
  uint16_t *w_router;
  float *act_clip;
  float act_sat_percentile;
  int32_t format;
} moe_w8a8_weights;

/* Optional per-stage outputs of moe_w8a8_forward for checking; every pointer
 * may be NULL. A = T*k. Rows of the permuted tensors are positions in the
 * expert-grouped order; entries past the number of kept rows (the last
 * expert_offsets value) are unspecified.
 *   topk_ids int32 [T][k], topk_w fp32 [T][k]  (routing result or the given ids)
 *   expert_counts int32 [E] kept rows per expert; expert_offsets int32 [E+1]
 *   sorted_assign int32 [A] assignment t*k+j of each permuted row
 *   row_of int32 [A] permuted row of assignment t*k+j, -1 if dropped
 *   qx int8 [T][H], sx fp32 [T]   per-token codes (e4m3 bytes in FP8 format)
 *                                 and scales
 *   acc1 int32 [A][2F]            GEMM1 accumulators (gate then up; the
 *                                 bits of the fp32 sums in FP8 format)
 *   h fp32 [A][F]                 SwiGLU output before requantisation
 *   qh int8 [A][F], sh fp32 [A]   requantised hidden rows and their scales
 *   y fp32 [A][H]                 dequantised down-projection rows, as the
 *                                 combine reads them */
typedef struct {
  int32_t *topk_ids;
  float *topk_w;
  int32_t *expert_counts;
  int32_t *expert_offsets;
  int32_t *sorted_assign;
  int32_t *row_of;
  int8_t *qx;
  float *sx;
  int32_t *acc1;
  float *h;
  int8_t *qh;
  float *sh;
  float *y;
  /* Kernel family of the two grouped GEMMs: 0 = chosen from the shape
   * (streaming kernels while experts average at most 32 rows, tiled kernels
   * beyond), 1 = streaming, 2 = tiled. Any other value: MOE_W8A8_ERR_INVALID.
   * Every choice computes the same result. */
  int32_t gemm_path;
  /* NULL, or an array of 18 hipEvent_t (as void*) to time the layer's
   * kernels on its own stream: entries 2s and 2s+1 are stamped with the
   * start and the end of the execution of the launch that performs stage s
   * (s = 0 route, 1 scan, 2 scatter, 3 activation quant, 4 GEMM1, 5 requant,
   * 6 GEMM2, 7 combine, 8 router projection), by that launch's own dispatch
   * (hipExtLaunchKernel), so timing inserts nothing between the kernels.
   * Stages fused into one launch are timed by the pair of the first of them:
   * for T*k <= 2048, stages 0-3 are one launch and pairs 1-3 are left
   * untouched. NULL entries are skipped. */
  void **stage_events;
  /* fp32 [T][E]: the router logits the routing used (the projection's
   * result in router-projection mode, a copy of router_logits otherwise;
   * untouched in pre-routed mode). */
  float *router_logits;
} moe_w8a8_debug;

/* Bytes of device workspace that moe_w8a8_forward needs for T tokens, and
 * that moe_w8a8_calibrate needs (T = 0 gives at least the calibrate size).
 * The caller allocates it once and hands it to every call
 * ("MiniMax-M3 W8A8 inference on K100AI" §4.3: reuse device memory from a
 * pool instead of allocating per call); the library allocates nothing.
 * A pure function of the arguments, nondecreasing in T (a workspace sized for
 * the largest batch serves every smaller one); returns 0 for invalid or
 * unsupported dimensions, T < 0, or a batch past the row limit of
 * moe_w8a8_forward. */
size_t moe_w8a8_workspace_size(const moe_w8a8_dims *dims, int64_t T);

/* Calibrate and quantise the layer weights ("MiniMax-M3 W8A8 inference on
 * K100AI" §3.2: SmoothQuant, per-channel weights; published SmoothQuant scale).
 *   alpha      migration strength in [0, 1] (the page's default is 0.6).
 *   calib_x    bf16 [n_calib][H] calibration tokens, n_calib >= 0.
 *   w_gate, w_up fp32 [E][F][H]; w_down fp32 [E][H][F] (unquantised, row-major).
 *   out        device buffers to fill (layouts above); the struct itself is
 *              host memory.
 * Computes, per input channel j: ax_j = max |calib_x[:, j]|,
 * aw_j = max over all experts and both projections of |W_gate|, |W_up| in
 * column j, s_j = ax_j^alpha / aw_j^(1-alpha) evaluated in fp64 and rounded to
 * fp32 (s_j = 1 when ax_j or aw_j is 0), inv_s_j = 1/s_j in fp32; then the
 * gate/up rows W[n][j] * s_j (fp32) and the down rows are quantised per row:
 * a = max |row|, code = rint(v * fl32(127/a)) clamped to [-127, 127],
 * scale = a/127 (an all-zero row gets scale 0 and codes 0).
 * Workspace: at least moe_w8a8_workspace_size(dims, 0) bytes.
 * Errors: MOE_W8A8_ERR_INVALID (NULL pointer, alpha outside [0,1],
 * n_calib < 0 or n_calib * H >= 2^61), MOE_W8A8_ERR_UNSUPPORTED, MOE_W8A8_ERR_WORKSPACE,
 * MOE_W8A8_ERR_HIP. */
int moe_w8a8_calibrate(const moe_w8a8_dims *dims, float alpha,
                       const uint16_t *calib_x, int64_t n_calib,
                       const float *w_gate, const float *w_up, const float *w_down,
                       const moe_w8a8_weights *out,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Static activation clipping threshold ("一晚上完成MoE模型推理优化…" §3.2:
 * the calibration clips activations beyond the 99.9th percentile of their
 * range). Writes act_clip[0] = the nearest-rank percentile `percentile` of
 * |fl32(calib_x[n][j] * inv_smooth[j])| over all n_calib * H entries: the
 * value of rank ceil(percentile/100 * N) (evaluated in fp64, clamped to
 * [1, N]) in ascending order; 0 when n_calib = 0.
 *   percentile in (0, 100]; calib_x bf16 [n_calib][H]; inv_smooth fp32 [H]
 *   (from moe_w8a8_calibrate); act_clip fp32 [1]. All device memory.
 * Errors: MOE_W8A8_ERR_INVALID (also n_calib * H >= 2^61),
 * MOE_W8A8_ERR_UNSUPPORTED, MOE_W8A8_ERR_HIP. */
int moe_w8a8_calibrate_clip(const moe_w8a8_dims *dims, float percentile,
                            const uint16_t *calib_x, int64_t n_calib,
                            const float *inv_smooth, float *act_clip, void *stream);

/* Forward pass of the layer for T tokens (steps 1-6 above).
 *   x           bf16 [T][H] input tokens.
 *   Routing input, one of three modes:
 *   router_logits fp32 [T][E] given; or
 *   topk_ids    int32 [T][k] and topk_w fp32 [T][k] (pre-routed mode): the
 *               assignments and their weights (ids outside [0, E) are treated
 *               as dropped; the weights are used as given; an expert named in
 *               several slots of a token gets one row per slot, each weighted
 *               by its own slot's weight and counted against the capacity); or
 *   neither (router-projection mode): the logits are x . w_router^T from
 *               weights->w_router, as moe_w8a8_router_logits computes them,
 *               and the routing of step 1 is taken on them.
 *   Giving router_logits together with topk_ids or topk_w, only one of
 *   topk_ids and topk_w, or neither with w_router NULL is an error.
 *   capacity_factor  > 0: each expert keeps at most
 *               C = ceil(capacity_factor * T * k / E) assignments (evaluated
 *               in fp64), the first C in (token, slot) order; dropped slots
 *               contribute nothing and the remaining weights are not
 *               renormalised. <= 0: no limit.
 *   out         bf16 [T][H] layer output (written for every token; a token
 *               whose every slot was dropped gets zeros).
 *   workspace   at least moe_w8a8_workspace_size(dims, T) bytes; contents on
 *               entry are ignored.
 *   debug       NULL, or a host struct of optional device outputs (above).
 * T == 0 is a successful no-op whatever the other pointers are (empty
 * tensors may carry NULL addresses). Errors: MOE_W8A8_ERR_INVALID (NULL required
 * pointer, T < 0, T*k >= 2^31 or T*k + 15*min(T*k, E) >= 2^31 (the permuted
 * rows with every expert group padded to 16), routing inputs as above, act_sat_percentile
 * outside {0} and (0, 100]), MOE_W8A8_ERR_UNSUPPORTED (also a saturation
 * rank m > 16), MOE_W8A8_ERR_WORKSPACE, MOE_W8A8_ERR_HIP. */
int moe_w8a8_forward(const moe_w8a8_dims *dims, const moe_w8a8_weights *weights,
                     const uint16_t *x, int64_t T,
                     const float *router_logits,
                     const int32_t *topk_ids, const float *topk_w,
                     float capacity_factor,
                     uint16_t *out,
                     void *workspace, size_t workspace_bytes,
                     const moe_w8a8_debug *debug, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * forward as moe_w8a8_forward, same arguments and results, but its workspace
 * is a static device array of MOE_W8A8_SCRATCH_BYTES inside the library (one
 * per GPU, held from the first call on that GPU until the process ends)
 * instead of a caller buffer. Nothing is allocated or freed by the call.
 * Limit: moe_w8a8_workspace_size(dims, T) <= MOE_W8A8_SCRATCH_BYTES (64 MiB:
 * e.g. up to ~220 tokens of a hidden-4096, 64-expert, top-8, FFN-1536 layer);
 * a larger batch returns MOE_W8A8_ERR_SCRATCH with nothing enqueued.
 * Every call on one GPU uses that GPU's one array, so calls that overlap on a
 * GPU (concurrent streams, or host threads) race and must be serialised by
 * the caller; consecutive calls on one stream are safe (each call's kernels
 * ignore what the array held before). Errors: as moe_w8a8_forward, with
 * MOE_W8A8_ERR_SCRATCH in place of MOE_W8A8_ERR_WORKSPACE. */
#define MOE_W8A8_SCRATCH_BYTES ((size_t)64 << 20)
int moe_w8a8_forward_noalloc(const moe_w8a8_dims *dims, const moe_w8a8_weights *weights,
                             const uint16_t *x, int64_t T,
                             const float *router_logits,
                             const int32_t *topk_ids, const float *topk_w,
                             float capacity_factor,
                             uint16_t *out,
                             const moe_w8a8_debug *debug, void *stream);

/* Router projection ("超大规模模型推理的Day0适配实践" §四: the gate belongs to
 * the fused MoE operator and the top-k it feeds must be exact; "MiniMax-M3
 * W8A8 inference on K100AI" §6.1: the routing layers stay in 16-bit float):
 *   logits[t][e] = sum_j x[t][j] * w_router[e][j]
 * with x bf16 [T][H], w_router bf16 [E][H] (device), accumulated in fp32 on
 * the bf16 matrix instructions (each product exact), written to logits fp32
 * [T][E] (device). The order of the sum depends on H only, never on T: H
 * is cut into parts of 512 channels, each part into 4 runs of 128 summed
 * ((r0 + r1) + r2) + r3, and the parts are added in order; within a run the
 * matrix instructions accumulate 16 channels at a time. A token's logits are
 * therefore the same whatever batch it comes in.
 * Workspace: at least moe_w8a8_workspace_size(dims, T) bytes (the per-part
 * sums; none is needed when H <= 512).
 * T == 0 is a successful no-op. Errors: MOE_W8A8_ERR_INVALID (NULL pointer,
 * T < 0), MOE_W8A8_ERR_UNSUPPORTED, MOE_W8A8_ERR_WORKSPACE, MOE_W8A8_ERR_HIP. */
int moe_w8a8_router_logits(const moe_w8a8_dims *dims, const uint16_t *x, int64_t T,
                           const uint16_t *w_router, float *logits,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Pack row-major codes into the fragment-tiled layout of moe_w8a8_weights
 * ("MiniMax-M3 W8A8 inference on K100AI" §3.2-§3.3: weights quantised by an
 * offline tool are built into the engine's own layout), so that INT8 or FP8
 * codes quantised elsewhere can be loaded:
 *   src   int8 (or e4m3 bytes) [count][N][K], row-major, device memory;
 *   dst   int8 [count][N][K] in the fragment-tiled layout (matrix c at byte
 *         c*N*K), device memory, not overlapping src.
 * Per expert: w_gate_up is count = E, N = 2F (gate rows, then up rows),
 * K = H; w_down is count = E, N = H, K = F. The scales (s_gate_up, s_down)
 * and smooth/inv_smooth are plain arrays and need no packing.
 * Nothing is allocated; the copy is enqueued on `stream`.
 * Errors: MOE_W8A8_ERR_INVALID (NULL pointer, count, N or K <= 0, a pointer
 * not 16-byte aligned, overlapping buffers, more than 2^40 bytes),
 * MOE_W8A8_ERR_UNSUPPORTED (N % 16 != 0 or K % 64 != 0), MOE_W8A8_ERR_HIP. */
int moe_w8a8_pack(int64_t count, int32_t N, int32_t K, const int8_t *src, int8_t *dst,
                  void *stream);

/* Static description of a return code (never NULL). */
const char *moe_w8a8_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W8A8_H */
