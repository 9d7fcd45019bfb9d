/* A C client of the library, with no Python and no torch: it reads a layer's
 * unquantised weights, calibration tokens, input tokens and router logits
 * from raw files, places them in device memory with hipMalloc, calibrates the
 * layer (moe_w8a8_calibrate), runs one forward (moe_w8a8_forward) on a stream
 * of its own and writes the bf16 output. Used by tests/test_gpu_c_client.py,
 * which compares that output with the same layer run through the Python
 * binding.
 *
 * usage: c_client DIR H F E K T N_CALIB ALPHA
 *   DIR/calib_x.bin  bf16 bits [N_CALIB][H]
 *   DIR/w_gate.bin, DIR/w_up.bin  fp32 [E][F][H]; DIR/w_down.bin fp32 [E][H][F]
 *   DIR/x.bin        bf16 bits [T][H];  DIR/logits.bin fp32 [T][E]
 *   writes DIR/out.bin  bf16 bits [T][H]
 */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "moe_w8a8.h"

static int fail(const char *what) {
  fprintf(stderr, "c_client: %s\n", what);
  return 1;
}

/* Reads exactly n bytes of DIR/name into a new device buffer. */
static void *upload(const char *dir, const char *name, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) return NULL;
  void *h = malloc(n ? n : 1);
  void *d = NULL;
  const int ok = h && fread(h, 1, n, f) == n && hipMalloc(&d, n ? n : 1) == hipSuccess &&
                 hipMemcpy(d, h, n, hipMemcpyHostToDevice) == hipSuccess;
  fclose(f);
  free(h);
  return ok ? d : NULL;
}

static void *device(size_t n) {
  void *d = NULL;
  return hipMalloc(&d, n ? n : 1) == hipSuccess ? d : NULL;
}

int main(int argc, char **argv) {
  if (argc != 9) return fail("usage: c_client DIR H F E K T N_CALIB ALPHA");
  const char *dir = argv[1];
  moe_w8a8_dims d;
  d.hidden = atoi(argv[2]);
  d.ffn = atoi(argv[3]);
  d.num_experts = atoi(argv[4]);
  d.top_k = atoi(argv[5]);
  const int64_t T = atol(argv[6]), nc = atol(argv[7]);
  const float alpha = (float)atof(argv[8]);
  const size_t H = (size_t)d.hidden, F = (size_t)d.ffn, E = (size_t)d.num_experts;

  uint16_t *calib_x = upload(dir, "calib_x.bin", (size_t)nc * H * 2);
  float *w_gate = upload(dir, "w_gate.bin", E * F * H * 4);
  float *w_up = upload(dir, "w_up.bin", E * F * H * 4);
  float *w_down = upload(dir, "w_down.bin", E * H * F * 4);
  uint16_t *x = upload(dir, "x.bin", (size_t)T * H * 2);
  float *logits = upload(dir, "logits.bin", (size_t)T * E * 4);
  if (!calib_x || !w_gate || !w_up || !w_down || !x || !logits) return fail("inputs");

  moe_w8a8_weights w;
  w.w_gate_up = device(E * 2 * F * H);
  w.w_down = device(E * H * F);
  w.s_gate_up = device(E * 2 * F * 4);
  w.s_down = device(E * H * 4);
  w.smooth = device(H * 4);
  w.inv_smooth = device(H * 4);
  w.w_router = NULL;
  w.act_clip = NULL;
  w.act_sat_percentile = 0.0f;
  w.format = MOE_W8A8_FORMAT_INT8;
  const size_t ws0 = moe_w8a8_workspace_size(&d, 0), wsT = moe_w8a8_workspace_size(&d, T);
  const size_t ws_bytes = ws0 > wsT ? ws0 : wsT;
  void *ws = device(ws_bytes);
  uint16_t *out = device((size_t)T * H * 2);
  if (!w.w_gate_up || !w.w_down || !w.s_gate_up || !w.s_down || !w.smooth || !w.inv_smooth ||
      !ws || !out || ws_bytes == 0)
    return fail("device buffers");

  hipStream_t st;
  if (hipStreamCreate(&st) != hipSuccess) return fail("stream");
  int rc = moe_w8a8_calibrate(&d, alpha, calib_x, nc, w_gate, w_up, w_down, &w, ws, ws_bytes, st);
  if (rc != MOE_W8A8_OK) return fail(moe_w8a8_strerror(rc));
  rc = moe_w8a8_forward(&d, &w, x, T, logits, NULL, NULL, 0.0f, out, ws, ws_bytes, NULL, st);
  if (rc != MOE_W8A8_OK) return fail(moe_w8a8_strerror(rc));
  if (hipStreamSynchronize(st) != hipSuccess) return fail("synchronize");

  const size_t n = (size_t)T * H * 2;
  void *h = malloc(n ? n : 1);
  if (!h || hipMemcpy(h, out, n, hipMemcpyDeviceToHost) != hipSuccess) return fail("download");
  char path[4096];
  snprintf(path, sizeof path, "%s/out.bin", dir);
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(h, 1, n, f) != n) return fail("write");
  fclose(f);
  free(h);
  printf("c_client ok: T=%ld H=%d E=%d k=%d\n", (long)T, d.hidden, d.num_experts, d.top_k);
  return 0;
}
