/*
 * moe_oracle.c -- plain CPU definition of the W8A8 MoE expert layer.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the oracle that the HIP path is
 * checked against. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the product path never does, and it shares
 * no code, header, table or helper with the HIP library.
 *
 * Every stage is written as the plain definition, one output at a time, with
 * no blocking, fusion or reordering. OpenMP only splits independent outputs
 * across threads; it never changes the order of any sum.
 *
 * Pages cited (titles as printed, or the address where the page has none):
 *   [K100AI]  "MiniMax-M3 W8A8 inference on K100AI" (mhpq.cn/news/1068415)
 *   [Opus-K3] "一晚上完成MoE模型推理优化：量化+算子融合，吞吐提升230%" (gtnt.cn/news/142538)
 *   [Day0]    "超大规模模型推理的Day0适配实践" (service.ruibaoantu.com, id 9569169)
 * The pages give the method in prose only. Where they leave a step open, the
 * reading taken here is stated at the function and listed with the others in
 * the design notes of the repository.
 *
 * Precision. Where floating point decides an integer (a quantised code, a
 * top-k choice) the decision is taken in fp32, the precision the device
 * kernels use; every other real-valued quantity (dequantised GEMM outputs,
 * SwiGLU, routing weights, the combine sum) is computed in fp64 from the exact
 * fp32/int inputs and rounded once at the end.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -shared -fPIC -lm
 * (no fast-math: rintf must round half to even and products must round to fp32).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- helpers */

static float bf16_bits_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round a double to the nearest bfloat16, ties to even, in one rounding step.
 * bfloat16 keeps fp32's exponent range and 8 significant bits, so the value is
 * rounded to a multiple of its quantum 2^(e-8) (2^-133 for subnormals). */
uint16_t oracle_f64_to_bf16(double v) {
  if (isnan(v)) return (uint16_t)0x7FC0;
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  uint16_t sign = (uint16_t)(neg ? 0x8000 : 0);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);                     /* a = m * 2^e, m in [0.5, 1) */
  int q = e - 8;                    /* quantum exponent for 8 significant bits */
  if (q < -133) q = -133;           /* subnormal range of bfloat16 */
  double r = rint(ldexp(a, -q));    /* exact scaling, then ties-to-even */
  double rv = ldexp(r, q);          /* representable in fp32 by construction */
  if (rv > 3.3895313892515355e38) return (uint16_t)(sign | 0x7F80); /* overflow -> inf */
  float f = (float)rv;              /* exact: rv has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFF));
}

/* Symmetric per-row INT8 quantiser with the fp32 decision rule.
 *
 * [K100AI §1.2, §3.2]: weights are quantised per output channel from their
 * range, activations per token, both to 8 bits. Readings: symmetric absmax
 * scaling; codes lie in [-127, 127] (symmetric, -128
 * unused); rounding is half to even; the code is rint(v * (127/amax)) with both
 * the reciprocal and the product rounded to fp32; the stored scale is
 * amax/127; an all-zero row gets scale 0 and codes 0. */
/* The quantiser at a given level (the row's range): codes for |v| above the
 * level saturate at +-127. quant_row below uses level = max |v|. */
static void quant_row_at(const float *v, int64_t n, float amax, int8_t *q, float *scale) {
  if (amax == 0.0f) {
    memset(q, 0, (size_t)n);
    *scale = 0.0f;
    return;
  }
  float rr = 127.0f / amax;
  for (int64_t i = 0; i < n; ++i) {
    float t = v[i] * rr;
    float c = rintf(t);
    if (c > 127.0f) c = 127.0f;
    if (c < -127.0f) c = -127.0f;
    q[i] = (int8_t)c;
  }
  *scale = amax / 127.0f;
}

static float row_absmax(const float *v, int64_t n) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf(v[i]);
    if (a > amax) amax = a;
  }
  return amax;
}

static void quant_row(const float *v, int64_t n, int8_t *q, float *scale) {
  quant_row_at(v, n, row_absmax(v, n), q, scale);
}

/* ---------------------------------------------------------------- FP8 */

/* OCP FP8 e4m3 ("fn"). [Day0 §二.1]: expert layers are stored in FP8 or INT8;
 * [Day0 §四]: activations follow the weights' format. Reading: the OCP e4m3
 * encoding (the one the gfx950 matrix instructions take): sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6);
 * the code 0x7f (and 0xff) is NaN, there is no infinity, the largest finite
 * value is 1.75 * 2^8 = 448. The code of a value is its nearest e4m3 value,
 * ties to the even code, with the sign bit of the value (so -0.0 -> 0x80);
 * values are clamped to [-448, 448] before, so nothing rounds past 448. */
double oracle_e4m3_value(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  return s ? -v : v;
}

uint8_t oracle_e4m3_code(float t) {
  const uint8_t sign = signbit(t) ? 0x80 : 0x00;
  const double a = fabs((double)t);  /* <= 448 */
  if (a < ldexp(1.0, -6)) {          /* subnormal binade: steps of 2^-9 */
    const double q = rint(ldexp(a, 9));   /* 0..8; 8 is the smallest normal */
    return sign | (uint8_t)q;
  }
  int ex;
  frexp(a, &ex);                     /* a in [2^(ex-1), 2^ex) */
  const int e = ex - 1;              /* unbiased exponent */
  double q = rint(ldexp(a, 3 - e));  /* 8..16 steps of 2^(e-3) */
  int eb = e + 7;
  if (q == 16.0) { q = 8.0; ++eb; }
  return sign | (uint8_t)((eb << 3) | ((int)q - 8));
}

/* The quantiser of either format at a given level. INT8: quant_row_at.
 * FP8: rr = fl32(448/level), code = e4m3 of clamp(fl32(v*rr), -448, 448),
 * scale = level/448; a zero level gives rr = 0 (codes of +-0) and scale 0. */
static void quant_row_fmt_at(const float *v, int64_t n, float level, int32_t fmt, int8_t *q,
                             float *scale) {
  if (fmt == 0) {
    quant_row_at(v, n, level, q, scale);
    return;
  }
  const float rr = level > 0.0f ? 448.0f / level : 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float t = v[i] * rr;
    t = fminf(fmaxf(t, -448.0f), 448.0f);
    q[i] = (int8_t)oracle_e4m3_code(t);
  }
  *scale = level / 448.0f;
}

static void quant_row_fmt(const float *v, int64_t n, int32_t fmt, int8_t *q, float *scale) {
  quant_row_fmt_at(v, n, row_absmax(v, n), fmt, q, scale);
}

/* Decoded value of every FP8 code (oracle_e4m3_value of it), filled once
 * when the library is loaded, so that a product's operands are looked up
 * rather than decoded again for every product. */
static double e4m3_values[256];
__attribute__((constructor)) static void fill_e4m3_values(void) {
  for (int c = 0; c < 256; ++c) e4m3_values[c] = oracle_e4m3_value((uint8_t)c);
}

/* Code value: INT8 codes as integers, FP8 codes decoded. */
static double code_value(int8_t c, int32_t fmt) {
  return fmt == 0 ? (double)c : e4m3_values[(uint8_t)c];
}

/* Exported forms used by the pins: rows of either format. */
void oracle_quant_rows_fmt(int64_t rows, int64_t n, const float *v, int32_t fmt, int8_t *q,
                           float *scale) {
  for (int64_t r = 0; r < rows; ++r) quant_row_fmt(v + r * n, n, fmt, q + r * n, scale + r);
}

/* Exported form of the quantiser, one row after another (used by the pins). */
void oracle_quant_rows(int64_t rows, int64_t n, const float *v, int8_t *q, float *scale) {
  for (int64_t r = 0; r < rows; ++r) quant_row(v + r * n, n, q + r * n, scale + r);
}

/* ------------------------------------------------------------- calibrate */

/* SmoothQuant calibration followed by per-output-channel weight quantisation.
 *
 * [K100AI §3.2]: quantisation config W8/A8, per_channel weights, per_token
 * activations, smooth_quant enabled with alpha 0.6; SmoothQuant moves part of
 * the activation range into the weights by an equivalent rescaling, alpha sets
 * how much. The formula is the published SmoothQuant one (Xiao et al.):
 *   s_j = max|X_j|^alpha / max|W_j|^(1-alpha)     (per input channel j)
 *   X' = X diag(s)^-1,  W' = W diag(s)  (W' multiplies the same input channel)
 * Readings: one s[H] for the whole layer, shared by every expert's gate and up
 * projections (they all consume the same token vector), so max|W_j| runs over
 * all experts and both projections; s is computed in fp64 and rounded once to
 * fp32; a channel with a zero activation or weight range keeps s = 1;
 * inv_s = 1/s in fp32; the down projection is not smoothed.
 *
 * Layouts (host, row-major): calib_x bf16 [n_calib][H]; w_gate, w_up fp32
 * [E][F][H]; w_down fp32 [E][H][F]. Outputs: s, inv_s [H]; q_gu int8
 * [E][2F][H] (rows 0..F-1 gate, F..2F-1 up); sw_gu [E][2F]; q_d int8 [E][H][F];
 * sw_d [E][H]. ws_gu (optional) receives the smoothed fp32 gate/up weights
 * [E][2F][H] before quantisation. */
int oracle_calibrate(int32_t H, int32_t F, int32_t E, float alpha,
                     const uint16_t *calib_x, int64_t n_calib,
                     const float *w_gate, const float *w_up, const float *w_down,
                     float *s, float *inv_s,
                     int8_t *q_gu, float *sw_gu, int8_t *q_d, float *sw_d,
                     float *ws_gu, int32_t fmt) {
  if (H <= 0 || F <= 0 || E <= 0 || n_calib < 0) return -1;
  double a = (double)alpha;
  #pragma omp parallel for schedule(static)
  for (int32_t j = 0; j < H; ++j) {
    float ax = 0.0f, aw = 0.0f;
    for (int64_t n = 0; n < n_calib; ++n) {
      float v = fabsf(bf16_bits_to_f32(calib_x[n * H + j]));
      if (v > ax) ax = v;
    }
    for (int32_t e = 0; e < E; ++e)
      for (int32_t f = 0; f < F; ++f) {
        float g = fabsf(w_gate[((int64_t)e * F + f) * H + j]);
        float u = fabsf(w_up[((int64_t)e * F + f) * H + j]);
        if (g > aw) aw = g;
        if (u > aw) aw = u;
      }
    float sj = 1.0f;
    if (ax > 0.0f && aw > 0.0f) sj = (float)(pow((double)ax, a) / pow((double)aw, 1.0 - a));
    s[j] = sj;
    inv_s[j] = 1.0f / sj;
  }
  #pragma omp parallel
  {
    float *row = (float *)malloc(sizeof(float) * (size_t)(H > F ? H : F));
    #pragma omp for schedule(static)
    for (int64_t r = 0; r < (int64_t)E * 2 * F; ++r) {
      int64_t e = r / (2 * F), n = r % (2 * F);
      const float *src = n < F ? w_gate + (e * F + n) * H : w_up + (e * F + (n - F)) * H;
      for (int32_t j = 0; j < H; ++j) row[j] = src[j] * s[j];
      if (ws_gu) memcpy(ws_gu + r * H, row, sizeof(float) * (size_t)H);
      quant_row_fmt(row, H, fmt, q_gu + r * H, sw_gu + r);
    }
    #pragma omp for schedule(static)
    for (int64_t r = 0; r < (int64_t)E * H; ++r)
      quant_row_fmt(w_down + r * F, F, fmt, q_d + r * F, sw_d + r);
    free(row);
  }
  return 0;
}

/* ----------------------------------------------------------------- route */

/* Softmax top-k routing with deterministic ties.
 *
 * [Day0 §四 (MoE operator fusion)]: the fused top-k must reproduce the
 * reference exactly, tie-break rule included; the rule taken here is that the
 * lower expert index wins. [Opus-K3 §1.1]: every MoE layer
 * routes each token to its top-k experts.
 * Definition: experts are ordered by (logit descending, index ascending) with
 * IEEE comparisons (so -0.0 and +0.0 tie); the first k are taken in that
 * order. Softmax is monotone, so selecting on logits equals selecting on
 * probabilities. Weights are the softmax over all experts restricted to the
 * chosen k and renormalised to sum to 1, which is
 *   w_j = exp(l_j - m) / sum_{i<k} exp(l_i - m),  m = largest chosen logit,
 * evaluated in fp64 and rounded to fp32. */
void oracle_route(int64_t T, int32_t E, int32_t k, const float *logits,
                  int32_t *ids, float *w) {
  #pragma omp parallel
  {
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    double *ex = (double *)malloc(sizeof(double) * (size_t)k);
    #pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const float *l = logits + t * E;
      memset(taken, 0, (size_t)E);
      for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e) {
          if (taken[e]) continue;
          if (best < 0 || l[e] > l[best]) best = e; /* strict: equal keeps the lower index */
        }
        taken[best] = 1;
        ids[t * k + j] = best;
      }
      double m = (double)l[ids[t * k]];
      double den = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        ex[j] = exp((double)l[ids[t * k + j]] - m);
        den += ex[j];
      }
      for (int32_t j = 0; j < k; ++j) w[t * k + j] = (float)(ex[j] / den);
    }
    free(taken);
    free(ex);
  }
}

/* Router projection. [Day0 §四]: the gate (the router's linear map) is the
 * first operator of the fused MoE operator; [K100AI §6.1]: the layers at the
 * routing stay in 16-bit floating point, not INT8. Reading: x bf16 [T][H],
 * router matrix bf16 [E][H]; the logits are the exact dot products
 *   logits[t][e] = sum_j x[t][j] * w[e][j],
 * evaluated in fp64 (each product of two bf16 values is exact; the sum of H
 * of them carries a relative error of about H * 2^-53). */
void oracle_router_logits(int64_t T, int32_t H, int32_t E, const uint16_t *x,
                          const uint16_t *w, double *logits) {
  #pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int32_t j = 0; j < H; ++j)
        acc += (double)bf16_bits_to_f32(x[t * H + j]) * (double)bf16_bits_to_f32(w[(int64_t)e * H + j]);
      logits[t * E + e] = acc;
    }
  }
}

/* --------------------------------------------------------------- permute */

/* Expert capacity. [Day0 §二.2]: the capacity factor bounds the tokens an
 * expert takes; too small drops tokens. Reading: C = ceil(cf * T * k / E)
 * evaluated in fp64; cf <= 0 means no limit (returned as 0). */
int64_t oracle_capacity(float cf, int64_t T, int32_t k, int32_t E) {
  if (!(cf > 0.0f)) return 0;
  return (int64_t)ceil((double)cf * (double)T * (double)k / (double)E);
}

/* Group assignments by expert ("sort" in [Day0 §四]).
 *
 * Assignment a = t*k + j sends token t to expert ids[a]. Scanning a in
 * increasing order, r = number of earlier assignments to the same expert; the
 * assignment is kept iff capacity <= 0 or r < capacity (the first C in
 * (token, slot) order stay, the rest are dropped). Kept groups are laid out
 * expert after expert (offsets = exclusive scan of kept counts) and, inside a
 * group, in (token, slot) order: row_of[a] = offsets[e] + r, sorted[row] = a.
 * A dropped assignment gets row_of = -1. Ids outside [0, E) are dropped too.
 * counts[e] is the kept count. Returns the number of kept rows. */
int64_t oracle_permute(int64_t T, int32_t E, int32_t k, const int32_t *ids, int64_t capacity,
                       int32_t *counts, int32_t *offsets, int32_t *sorted, int32_t *row_of) {
  int64_t A = T * k;
  int64_t *seen = (int64_t *)calloc((size_t)E, sizeof(int64_t));
  int64_t *rank = (int64_t *)malloc(sizeof(int64_t) * (size_t)(A > 0 ? A : 1));
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t a = 0; a < A; ++a) {
    int32_t e = ids[a];
    if (e < 0 || e >= E) { rank[a] = -1; continue; }
    int64_t r = seen[e]++;
    if (capacity <= 0 || r < capacity) { rank[a] = r; counts[e] += 1; }
    else rank[a] = -1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  for (int64_t a = 0; a < A; ++a) {
    if (rank[a] < 0) { row_of[a] = -1; continue; }
    int32_t row = offsets[ids[a]] + (int32_t)rank[a];
    row_of[a] = row;
    sorted[row] = (int32_t)a;
  }
  int64_t kept = offsets[E];
  free(seen);
  free(rank);
  return kept;
}

/* ------------------------------------------------------ activation clips */

/* Nearest-rank percentile. [Opus-K3 §3.2]: the calibration truncates
 * activation values beyond the 99.9th percentile of their range (a range set
 * by the extremes stretches the step and costs the small values precision).
 * Reading: for N values sorted ascending, the p-th percentile is the value
 * of rank r = ceil(p / 100 * N) (1-based, evaluated in fp64, clamped to
 * [1, N]); no interpolation, so the threshold is one of the data values. */
static int cmp_float(const void *a, const void *b) {
  const float x = *(const float *)a, y = *(const float *)b;
  return (x > y) - (x < y);
}

int64_t oracle_percentile_rank(double p, int64_t N) {
  int64_t r = (int64_t)ceil(p / 100.0 * (double)N);
  if (r < 1) r = 1;
  if (r > N) r = N;
  return r;
}

/* Static clipping threshold over the calibration tokens, taken on the
 * smoothed activations the forward quantises: c = percentile p of
 * |fl32(x[n][j] * inv_s[j])| over all n_calib * H entries. 0 when there are no
 * entries. */
float oracle_clip_threshold(int64_t n_calib, int32_t H, const uint16_t *x, const float *inv_s,
                            float p) {
  const int64_t N = n_calib * (int64_t)H;
  if (N <= 0) return 0.0f;
  float *a = (float *)malloc(sizeof(float) * (size_t)N);
  for (int64_t n = 0; n < n_calib; ++n)
    for (int32_t j = 0; j < H; ++j) a[n * H + j] = fabsf(bf16_bits_to_f32(x[n * H + j]) * inv_s[j]);
  qsort(a, (size_t)N, sizeof(float), cmp_float);
  const float c = a[oracle_percentile_rank((double)p, N) - 1];
  free(a);
  return c;
}

/* Level at which a smoothed token row is quantised. [K100AI §6.4]: besides
 * per-token scales and SmoothQuant, activations may be saturated at a
 * threshold instead of stretching the scale to the row's maximum.
 *   clip > 0      static threshold (from the calibration above);
 *   sat_p in (0, 100]: dynamic threshold, the row's own nearest-rank
 *                 percentile sat_p of |v| (sorted copy of the row);
 * the level is the smallest of max |v| and the enabled thresholds that are
 * > 0 (a zero threshold, e.g. a mostly-zero row, leaves the level alone). */
static float clip_level(const float *v, int32_t n, float clip, float sat_p, float *tmp) {
  float level = row_absmax(v, n);
  if (clip > 0.0f && clip < level) level = clip;
  if (sat_p > 0.0f) {
    for (int32_t j = 0; j < n; ++j) tmp[j] = fabsf(v[j]);
    qsort(tmp, (size_t)n, sizeof(float), cmp_float);
    const float t = tmp[oracle_percentile_rank((double)sat_p, n) - 1];
    if (t > 0.0f && t < level) level = t;
  }
  return level;
}

/* ------------------------------------------------------------- act quant */

/* Per-token activation quantisation with the smoothing folded in.
 * [K100AI §3.2, §6.4]: activations are quantised per token (one outlier token
 * must not set the range of others) after SmoothQuant's rescaling.
 * xs_j = x_j * inv_s_j in fp32, then the quantiser above over the row. */
void oracle_act_quant_clip(int64_t T, int32_t H, const uint16_t *x, const float *inv_s,
                           float clip, float sat_p, int32_t fmt, int8_t *qx, float *sx) {
  #pragma omp parallel
  {
    float *row = (float *)malloc(sizeof(float) * (size_t)H);
    float *tmp = (float *)malloc(sizeof(float) * (size_t)H);
    #pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      for (int32_t j = 0; j < H; ++j) row[j] = bf16_bits_to_f32(x[t * H + j]) * inv_s[j];
      quant_row_fmt_at(row, H, clip_level(row, H, clip, sat_p, tmp), fmt, qx + t * H, sx + t);
    }
    free(row);
    free(tmp);
  }
}

void oracle_act_quant(int64_t T, int32_t H, const uint16_t *x, const float *inv_s,
                      int8_t *qx, float *sx) {
  oracle_act_quant_clip(T, H, x, inv_s, 0.0f, 0.0f, 0, qx, sx);
}

/* ------------------------------------------------------------ expert row */

/* One kept (token, expert) row through the expert FFN.
 *
 * [K100AI §1.2]: W8A8 multiplies INT8 weights by INT8 activations with integer
 * accumulation and dequantises the result. [K100AI §4.3]: consecutive matmuls
 * stay in the INT8 domain (the hidden activation is requantised, not kept in
 * float between the two projections). [Opus-K3 §4.1]: the activation that
 * follows a linear layer belongs with it. SwiGLU form: h = silu(gate) * up.
 *   acc1[n] = sum_j qx[j] * w_gu[n][j]                      (int32, exact)
 *   g = acc1[f] * sx * sw_gu[f],  u = acc1[F+f] * sx * sw_gu[F+f]   (fp64)
 *   h[f] = fl32( g / (1 + exp(-g)) * u )
 *   (qh, sh) = quantiser(h)             (per (token, expert) row, fp32 rule)
 *   acc2[n] = sum_f qh[f] * w_d[n][f]                       (int32, exact)
 *   y[n] = acc2[n] * sh * sw_d[n]                           (fp64)
 * acc1 and h may be NULL. */
void oracle_expert_row(int32_t H, int32_t F, const int8_t *qx_row, float sx,
                       const int8_t *q_gu_e, const float *sw_gu_e,
                       const int8_t *q_d_e, const float *sw_d_e, int32_t fmt,
                       int32_t *acc1, double *acc1f, float *h, int8_t *qh, float *sh, double *y) {
  /* acc: exact integer sums for INT8 codes (int32, |sum| <= K * 127^2), exact
   * fp64 sums of the decoded products for FP8 codes. */
  double *acc = (double *)malloc(sizeof(double) * (size_t)(2 * F));
  float *hf = (float *)malloc(sizeof(float) * (size_t)F);
  for (int32_t n = 0; n < 2 * F; ++n) {
    const int8_t *wr = q_gu_e + (int64_t)n * H;
    if (fmt == 0) {
      int32_t s = 0;
      for (int32_t j = 0; j < H; ++j) s += (int32_t)qx_row[j] * (int32_t)wr[j];
      acc[n] = (double)s;
    } else {
      double s = 0.0;
      for (int32_t j = 0; j < H; ++j) s += code_value(qx_row[j], fmt) * code_value(wr[j], fmt);
      acc[n] = s;
    }
  }
  for (int32_t f = 0; f < F; ++f) {
    double g = acc[f] * (double)sx * (double)sw_gu_e[f];
    double u = acc[F + f] * (double)sx * (double)sw_gu_e[F + f];
    hf[f] = (float)(g / (1.0 + exp(-g)) * u);
  }
  quant_row_fmt(hf, F, fmt, qh, sh);
  for (int32_t n = 0; n < H; ++n) {
    const int8_t *wr = q_d_e + (int64_t)n * F;
    double s = 0.0;
    if (fmt == 0) {
      int32_t si = 0;
      for (int32_t f = 0; f < F; ++f) si += (int32_t)qh[f] * (int32_t)wr[f];
      s = (double)si;
    } else {
      for (int32_t f = 0; f < F; ++f) s += code_value(qh[f], fmt) * code_value(wr[f], fmt);
    }
    y[n] = s * (double)(*sh) * (double)sw_d_e[n];
  }
  for (int32_t n = 0; n < 2 * F; ++n) {
    if (acc1) acc1[n] = (int32_t)acc[n];
    if (acc1f) acc1f[n] = acc[n];
  }
  if (h) memcpy(h, hf, sizeof(float) * (size_t)F);
  free(acc);
  free(hf);
}

/* The expert row for a list of permuted rows (row i = sorted position).
 * Row i belongs to assignment a = sorted[i], token t = a / k, expert
 * e = ids[a]. Outputs are indexed by position in `rows`. */
void oracle_expert_rows(int64_t nrows, const int32_t *rows, int32_t H, int32_t F, int32_t k,
                        const int32_t *ids, const int32_t *sorted,
                        const int8_t *qx, const float *sx,
                        const int8_t *q_gu, const float *sw_gu,
                        const int8_t *q_d, const float *sw_d, int32_t fmt,
                        int32_t *acc1, double *acc1f, float *h, int8_t *qh, float *sh,
                        double *y) {
  #pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    int32_t a = sorted[rows[r]];
    int64_t t = a / k;
    int64_t e = ids[a];
    oracle_expert_row(H, F, qx + t * H, sx[t],
                      q_gu + e * 2 * F * (int64_t)H, sw_gu + e * 2 * F,
                      q_d + e * (int64_t)H * F, sw_d + e * H, fmt,
                      acc1 ? acc1 + r * 2 * F : NULL, acc1f ? acc1f + r * 2 * F : NULL,
                      h ? h + r * F : NULL, qh + r * F, sh + r, y + r * H);
  }
}

/* ---------------------------------------------------------------- combine */

/* Gate-weighted un-permute and sum ("un-sort, weighted sum" in [Day0 §四]).
 * out[t][n] = bf16( sum over slots j with row_of[t*k+j] >= 0 of
 *                   w[t][j] * y[row_of[t*k+j]][n] ), summed in fp64 in slot
 * order and rounded once to bfloat16. A dropped slot contributes nothing and
 * the remaining weights are not renormalised. y_row_index maps a permuted row
 * to its row in y (NULL: identity). exact (may be NULL) receives the fp64 sum
 * itself, before the rounding to bfloat16. */
void oracle_combine(int64_t ntok, const int64_t *tokens, int32_t H, int32_t k,
                    const float *w, const int32_t *row_of, const int64_t *y_row_index,
                    const double *y, uint16_t *out, double *exact) {
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < ntok; ++i) {
    int64_t t = tokens ? tokens[i] : i;
    for (int32_t n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        int32_t row = row_of[t * k + j];
        if (row < 0) continue;
        int64_t yr = y_row_index ? y_row_index[row] : row;
        acc += (double)w[t * k + j] * y[yr * H + n];
      }
      out[i * (int64_t)H + n] = oracle_f64_to_bf16(acc);
      if (exact) exact[i * (int64_t)H + n] = acc;
    }
  }
}

/* ---------------------------------------------------------------- forward */

/* The whole layer: route (or take the pre-routed ids and weights), permute,
 * quantise the tokens, run every kept row through its expert, combine.
 * All buffers are host memory owned by the caller. logits == NULL selects
 * pre-routed mode (ids_in/w_in). acc1 and h may be NULL. Sizes: A = T*k;
 * ids, w, row_of [A]; counts [E]; offsets [E+1]; sorted, sh [A]; qx [T][H];
 * sx [T]; acc1 [A][2F]; h, qh [A][F]; y [A][H] (fp64); out [T][H] bf16;
 * out_exact [T][H] fp64 (may be NULL): the combine's sum before rounding.
 * Returns the number of kept rows. */
int64_t oracle_forward(int64_t T, int32_t H, int32_t F, int32_t E, int32_t k,
                       const uint16_t *x, const float *logits,
                       const int32_t *ids_in, const float *w_in, float capacity_factor,
                       const int8_t *q_gu, const float *sw_gu,
                       const int8_t *q_d, const float *sw_d, const float *inv_s,
                       float clip, float sat_p, int32_t fmt,
                       int32_t *ids, float *w, int32_t *counts, int32_t *offsets,
                       int32_t *sorted, int32_t *row_of, int8_t *qx, float *sx,
                       int32_t *acc1, double *acc1f, float *h, int8_t *qh, float *sh,
                       double *y, uint16_t *out, double *out_exact) {
  int64_t A = T * k;
  if (logits) oracle_route(T, E, k, logits, ids, w);
  else {
    memcpy(ids, ids_in, sizeof(int32_t) * (size_t)A);
    memcpy(w, w_in, sizeof(float) * (size_t)A);
  }
  int64_t cap = oracle_capacity(capacity_factor, T, k, E);
  int64_t kept = oracle_permute(T, E, k, ids, cap, counts, offsets, sorted, row_of);
  oracle_act_quant_clip(T, H, x, inv_s, clip, sat_p, fmt, qx, sx);
  int32_t *rows = (int32_t *)malloc(sizeof(int32_t) * (size_t)(kept > 0 ? kept : 1));
  for (int64_t i = 0; i < kept; ++i) rows[i] = (int32_t)i;
  oracle_expert_rows(kept, rows, H, F, k, ids, sorted, qx, sx, q_gu, sw_gu, q_d, sw_d, fmt,
                     acc1, acc1f, h, qh, sh, y);
  free(rows);
  oracle_combine(T, NULL, H, k, w, row_of, NULL, y, out, out_exact);
  return kept;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
