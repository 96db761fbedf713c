/* The whole hot path from plain C99, with no Python and no torch: device
 * buffers from the HIP runtime, then sparge_predict_mask and sparge_attn
 * through include/sparge.h on the default stream.
 *
 *   attn_from_c DIR B H H_KV N D CAUSAL TAU THETA LAMBDA
 *
 * reads DIR/q.bin ([B,H,N,D] bf16 bits), DIR/k.bin and DIR/v.bin
 * ([B,H_KV,N,D] bf16 bits), all contiguous, and writes DIR/mg.bin (uint8
 * [B,H,Tm,Tn]), DIR/o.bin (float32 [B,H,N,D]), DIR/counts.bin (int64[8])
 * and DIR/dbg.bin (the per-group lambda decisions, uint8
 * [B,H,Tm,Tn,SPARGE_BQ/rows per wavefront]).  Prints "ok" and returns 0, or
 * names the failed step and returns 1. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sparge.h"

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    printf("failed: %s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static int read_file(const char* dir, const char* name, void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) {
    printf("failed: cannot open %s\n", path);
    return 0;
  }
  size_t got = fread(buf, 1, bytes, f);
  fclose(f);
  if (got != bytes) printf("failed: %s holds %zu bytes, expected %zu\n", path, got, bytes);
  return got == bytes;
}

static int write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) {
    printf("failed: cannot create %s\n", path);
    return 0;
  }
  size_t put = fwrite(buf, 1, bytes, f);
  fclose(f);
  return put == bytes;
}

static sparge_tensor contiguous(int64_t B, int64_t H, int64_t N, int64_t d) {
  sparge_tensor t;
  t.B = B;
  t.H = H;
  t.N = N;
  t.d = d;
  t.sn = d;
  t.sh = N * d;
  t.sb = H * N * d;
  return t;
}

int main(int argc, char** argv) {
  if (argc != 11) {
    printf("usage: %s DIR B H H_KV N D CAUSAL TAU THETA LAMBDA\n", argv[0]);
    return 1;
  }
  const char* dir = argv[1];
  const int64_t B = atoll(argv[2]), H = atoll(argv[3]), Hkv = atoll(argv[4]), N = atoll(argv[5]),
                d = atoll(argv[6]);
  const int causal = atoi(argv[7]);
  const double tau = atof(argv[8]), theta = atof(argv[9]), lam = atof(argv[10]);
  const int64_t Tm = (N + SPARGE_BQ - 1) / SPARGE_BQ, Tn = (N + SPARGE_BK - 1) / SPARGE_BK;
  const int64_t groups = SPARGE_BQ / sparge_rows_per_wave();

  sparge_tensor qs = contiguous(B, H, N, d), ks = contiguous(B, Hkv, N, d);
  sparge_tensor vs = ks, os = qs;
  const size_t q_bytes = (size_t)(B * H * N * d) * 2, kv_bytes = (size_t)(B * Hkv * N * d) * 2;
  const size_t o_bytes = (size_t)(B * H * N * d) * 4, mg_bytes = (size_t)(B * H * Tm * Tn);
  const size_t dbg_bytes = mg_bytes * (size_t)groups;
  const size_t ws_bytes = sparge_workspace_size(&qs, &ks);
  if (ws_bytes == 0) {
    printf("failed: workspace size 0\n");
    return 1;
  }

  void *h_q = malloc(q_bytes), *h_k = malloc(kv_bytes), *h_v = malloc(kv_bytes);
  void *h_o = malloc(o_bytes), *h_mg = malloc(mg_bytes), *h_dbg = malloc(dbg_bytes);
  int64_t h_counts[SPARGE_NUM_COUNTERS];
  if (!h_q || !h_k || !h_v || !h_o || !h_mg || !h_dbg) {
    printf("failed: host allocation\n");
    return 1;
  }
  if (!read_file(dir, "q.bin", h_q, q_bytes) || !read_file(dir, "k.bin", h_k, kv_bytes) ||
      !read_file(dir, "v.bin", h_v, kv_bytes))
    return 1;

  void *q = NULL, *k = NULL, *v = NULL, *o = NULL, *ws = NULL;
  uint8_t *mg = NULL, *dbg = NULL;
  int32_t* row_cnt = NULL;
  uint16_t* row_idx = NULL;
  int64_t* counts = NULL;
  if (!hip_ok(hipMalloc(&q, q_bytes), "hipMalloc q") || !hip_ok(hipMalloc(&k, kv_bytes), "hipMalloc k") ||
      !hip_ok(hipMalloc(&v, kv_bytes), "hipMalloc v") || !hip_ok(hipMalloc(&o, o_bytes), "hipMalloc o") ||
      !hip_ok(hipMalloc(&ws, ws_bytes), "hipMalloc workspace") ||
      !hip_ok(hipMalloc((void**)&mg, mg_bytes), "hipMalloc mg") ||
      !hip_ok(hipMalloc((void**)&dbg, dbg_bytes), "hipMalloc dbg") ||
      !hip_ok(hipMalloc((void**)&row_cnt, (size_t)(B * H * Tm) * 4), "hipMalloc row_cnt") ||
      !hip_ok(hipMalloc((void**)&row_idx, mg_bytes * 2), "hipMalloc row_idx") ||
      !hip_ok(hipMalloc((void**)&counts, sizeof h_counts), "hipMalloc counts"))
    return 1;
  if (!hip_ok(hipMemcpy(q, h_q, q_bytes, hipMemcpyHostToDevice), "copy q") ||
      !hip_ok(hipMemcpy(k, h_k, kv_bytes, hipMemcpyHostToDevice), "copy k") ||
      !hip_ok(hipMemcpy(v, h_v, kv_bytes, hipMemcpyHostToDevice), "copy v") ||
      !hip_ok(hipMemset(dbg, 0, dbg_bytes), "clear dbg"))
    return 1;

  int r = sparge_predict_mask(q, &qs, k, &ks, SPARGE_BF16, tau, theta, causal, mg, row_cnt, row_idx, NULL, NULL,
                              ws, ws_bytes, NULL);
  if (r != SPARGE_OK) {
    printf("failed: sparge_predict_mask %d: %s\n", r, sparge_last_error());
    return 1;
  }
  r = sparge_attn(q, &qs, k, &ks, v, &vs, o, &os, SPARGE_BF16, SPARGE_BF16, SPARGE_F32, NULL, NULL, mg, row_cnt,
                  row_idx, lam, causal, counts, dbg, ws, ws_bytes, NULL);
  if (r != SPARGE_OK) {
    printf("failed: sparge_attn %d: %s\n", r, sparge_last_error());
    return 1;
  }
  if (!hip_ok(hipDeviceSynchronize(), "synchronize") ||
      !hip_ok(hipMemcpy(h_o, o, o_bytes, hipMemcpyDeviceToHost), "copy o") ||
      !hip_ok(hipMemcpy(h_mg, mg, mg_bytes, hipMemcpyDeviceToHost), "copy mg") ||
      !hip_ok(hipMemcpy(h_dbg, dbg, dbg_bytes, hipMemcpyDeviceToHost), "copy dbg") ||
      !hip_ok(hipMemcpy(h_counts, counts, sizeof h_counts, hipMemcpyDeviceToHost), "copy counts"))
    return 1;
  if (!write_file(dir, "o.bin", h_o, o_bytes) || !write_file(dir, "mg.bin", h_mg, mg_bytes) ||
      !write_file(dir, "dbg.bin", h_dbg, dbg_bytes) || !write_file(dir, "counts.bin", h_counts, sizeof h_counts))
    return 1;

  hipFree(q);
  hipFree(k);
  hipFree(v);
  hipFree(o);
  hipFree(ws);
  hipFree(mg);
  hipFree(dbg);
  hipFree(row_cnt);
  hipFree(row_idx);
  hipFree(counts);
  free(h_q);
  free(h_k);
  free(h_v);
  free(h_o);
  free(h_mg);
  free(h_dbg);
  printf("ok\n");
  return 0;
}
