/* One batch step from plain C through the C ABI on the GPU: reads a small batch
 * from binary files (written by tests/test_c_abi.py from the seeded generator),
 * copies it to the device with the HIP runtime, runs rpkv_prepare_metadata
 * (growing the workspace to the size the library reports) and rpkv_forward, and
 * writes the output and the K pool back.  Usage: abi_forward <dir>. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rpkv.h"

static void *slurp(const char *dir, const char *name, size_t *bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
  fseek(f, 0, SEEK_END);
  long n = ftell(f);
  fseek(f, 0, SEEK_SET);
  void *buf = malloc(n > 0 ? (size_t)n : 1);
  if (n > 0 && fread(buf, 1, (size_t)n, f) != (size_t)n) { fprintf(stderr, "short read\n"); exit(2); }
  fclose(f);
  *bytes = (size_t)n;
  return buf;
}

static void spill(const char *dir, const char *name, const void *buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(buf, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
  fclose(f);
}

#define HIP_OK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
  fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_)); return 3; } } while (0)
#define RPKV_OK_(x) do { rpkv_status s_ = (x); if (s_ != RPKV_OK) { \
  fprintf(stderr, "%s: %s: %s\n", #x, rpkv_status_string(s_), rpkv_last_error()); return 4; } } while (0)

static void *to_dev(const void *host, size_t bytes) {
  void *d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 16) != hipSuccess) return NULL;
  if (bytes && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

int main(int argc, char **argv) {
  if (argc != 2) { fprintf(stderr, "usage: abi_forward <dir>\n"); return 1; }
  const char *dir = argv[1];
  size_t nb;
  int32_t *meta = (int32_t *)slurp(dir, "meta.bin", &nb);
  /* Hq Hkv D P num_pages batch T cols */
  const int32_t Hq = meta[0], Hkv = meta[1], D = meta[2], P = meta[3], num_pages = meta[4];
  const int32_t batch = meta[5], T = meta[6], cols = meta[7];
  size_t b_cu, b_L, b_pt, b_sm, b_q, b_k, b_v, b_kp, b_vp;
  int32_t *cu = (int32_t *)slurp(dir, "cu.bin", &b_cu);
  int32_t *L = (int32_t *)slurp(dir, "L.bin", &b_L);
  int32_t *pt = (int32_t *)slurp(dir, "pt.bin", &b_pt);
  void *sm = slurp(dir, "sm.bin", &b_sm);
  void *q = slurp(dir, "q.bin", &b_q), *k = slurp(dir, "k.bin", &b_k), *v = slurp(dir, "v.bin", &b_v);
  void *kp = slurp(dir, "kpool.bin", &b_kp), *vp = slurp(dir, "vpool.bin", &b_vp);

  rpkv_shape s;
  memset(&s, 0, sizeof s);
  s.num_q_heads = Hq;
  s.num_kv_heads = Hkv;
  s.head_dim = D;
  s.page_size = P;
  s.dtype = RPKV_BF16;
  s.max_batch = batch;
  s.num_pages = num_pages;
  s.max_tokens = T;
  s.max_pages_per_req = cols;
  rpkv_plan *plan = NULL;
  RPKV_OK_(rpkv_plan_create(&s, &plan));

  void *d_pt = to_dev(pt, b_pt), *d_sm = to_dev(sm, b_sm), *d_q = to_dev(q, b_q);
  void *d_k = to_dev(k, b_k), *d_v = to_dev(v, b_v), *d_kp = to_dev(kp, b_kp), *d_vp = to_dev(vp, b_vp);
  void *d_out = NULL;
  HIP_OK(hipMalloc(&d_out, b_q));
  if (!d_pt || !d_sm || !d_q || !d_k || !d_v || !d_kp || !d_vp) { fprintf(stderr, "device copy failed\n"); return 3; }

  /* the first prepare reports the workspace the batch needs */
  void *ws = NULL;
  size_t ws_bytes = 0;
  rpkv_status st = rpkv_prepare_metadata(plan, batch, cu, L, (const int32_t *)d_pt, cols, cols, pt,
                                         NULL, 0, ws, ws_bytes, NULL);
  if (st == RPKV_ERR_WORKSPACE_TOO_SMALL) {
    RPKV_OK_(rpkv_workspace_bytes(plan, &ws_bytes));
    HIP_OK(hipMalloc(&ws, ws_bytes));
    st = rpkv_prepare_metadata(plan, batch, cu, L, (const int32_t *)d_pt, cols, cols, pt, NULL, 0,
                               ws, ws_bytes, NULL);
  }
  RPKV_OK_(st);
  const float scale = 1.0f / __builtin_sqrtf((float)D);
  RPKV_OK_(rpkv_forward(plan, d_q, d_k, d_v, (const int32_t *)d_sm, d_kp, d_vp, d_out, scale, NULL));
  HIP_OK(hipDeviceSynchronize());

  void *out = malloc(b_q);
  HIP_OK(hipMemcpy(out, d_out, b_q, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(kp, d_kp, b_kp, hipMemcpyDeviceToHost));
  spill(dir, "out.bin", out, b_q);
  spill(dir, "kpool_after.bin", kp, b_kp);
  rpkv_plan_destroy(plan);
  printf("ok workspace %zu\n", ws_bytes);
  return 0;
}
