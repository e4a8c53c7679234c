/*
 * swa_c_check.c — the C ABI driven from plain C (no Python, no torch): a
 * prefill chunk without a cache, the cache write of the chunk, then three
 * fused decode steps, on HIP device buffers the program allocates itself.
 * The inputs come from a 32-bit linear congruential generator (multiplier
 * 1664525, increment 1013904223), each value (state >> 8) / 2^24 * 2 - 1
 * rounded to bf16 to nearest even, so that a test can rebuild them.  The
 * outputs and the final caches are written, as raw bytes in that order, to
 * the file named by argv[1].  Exit status 0 on success; on an error the
 * failing call and its status string go to stderr.
 *
 * Built by sliding_window_gqa_amd/build.py with gcc against include/swa.h and
 * libswa.so; run by tests/test_gpu_c_abi.py.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "swa.h"

enum { B = 2, HQ = 8, HKV = 2, D = 128, W = 128, C = 200, STEPS = 3 };

static uint32_t lcg = 12345u;

static uint16_t next_bf16(void) {
  lcg = lcg * 1664525u + 1013904223u;
  float f = (float)(lcg >> 8) * (1.0f / 16777216.0f) * 2.0f - 1.0f;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void* dev_fill(size_t n) {   /* n bf16 values from the generator, on the device */
  uint16_t* h = (uint16_t*)malloc(n * sizeof(uint16_t));
  void* d = NULL;
  if (!h) return NULL;
  for (size_t i = 0; i < n; ++i) h[i] = next_bf16();
  if (hipMalloc(&d, n * sizeof(uint16_t)) != hipSuccess ||
      hipMemcpy(d, h, n * sizeof(uint16_t), hipMemcpyHostToDevice) != hipSuccess)
    d = NULL;
  free(h);
  return d;
}

static void* dev_alloc(size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes) != hipSuccess) return NULL;
  if (hipMemset(d, 0, bytes) != hipSuccess) return NULL;
  return d;
}

static int dump(FILE* f, const void* d, size_t bytes) {
  void* h = malloc(bytes);
  int ok = h && hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost) == hipSuccess &&
           fwrite(h, 1, bytes, f) == bytes;
  free(h);
  return ok;
}

#define CHECK(call)                                                              \
  do {                                                                           \
    int st_ = (call);                                                            \
    if (st_ != SWA_OK) {                                                         \
      fprintf(stderr, "%s -> %s\n", #call, swa_status_string(st_));              \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUTPUT_FILE\n", argv[0]);
    return 2;
  }
  swa_params p;
  memset(&p, 0, sizeof p);
  p.batch = B;
  p.n_q_heads = HQ;
  p.n_kv_heads = HKV;
  p.head_dim = D;
  p.window = W;
  p.n_sink = 0;
  p.scale = 0.0f;        /* 1/sqrt(head_dim) */
  p.rope_theta = 10000.0f;
  p.dtype = SWA_BF16;
  p.dilation = 1;

  const size_t nq = (size_t)B * C * HQ * D, nk = (size_t)B * C * HKV * D;
  void* q = dev_fill(nq);
  void* k = dev_fill(nk);
  void* v = dev_fill(nk);
  const size_t cache_bytes = (size_t)B * W * HKV * D * 2;
  void* kc = dev_alloc(cache_bytes);
  void* vc = dev_alloc(cache_bytes);
  void* out = dev_alloc(nq * 2);
  void* lse = dev_alloc((size_t)B * HQ * C * 4);
  const size_t ws_bytes = swa_prefill_workspace_bytes(&p, C);
  const size_t dws_bytes = swa_decode_workspace_bytes(&p);
  void* ws = dev_alloc(ws_bytes);
  void* dws = dev_alloc(dws_bytes);
  int32_t h_start[B] = {0, 0};
  int32_t* start = (int32_t*)dev_alloc(sizeof h_start);
  if (!q || !k || !v || !kc || !vc || !out || !lse || !ws || !dws || !start || ws_bytes == 0 ||
      dws_bytes == 0 || hipMemcpy(start, h_start, sizeof h_start, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "device allocation or copy failed\n");
    return 1;
  }
  FILE* f = fopen(argv[1], "wb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 1;
  }

  /* the first chunk (no position before it), then its cache write */
  CHECK(swa_prefill_chunk(&p, q, k, v, NULL, NULL, start, C, out, (float*)lse, ws, ws_bytes, 0));
  CHECK(swa_cache_write(&p, k, v, start, C, kc, vc, 0));
  if (hipDeviceSynchronize() != hipSuccess || !dump(f, out, nq * 2) ||
      !dump(f, lse, (size_t)B * HQ * C * 4)) {
    fprintf(stderr, "prefill readback failed\n");
    return 1;
  }

  /* decode steps at positions C, C+1, ... (write + attention in one call) */
  const size_t n1q = (size_t)B * HQ * D, n1k = (size_t)B * HKV * D;
  void* out1 = dev_alloc(n1q * 2);
  void* lse1 = dev_alloc((size_t)B * HQ * 4);
  int32_t* pos = (int32_t*)dev_alloc(B * sizeof(int32_t));
  for (int s = 0; s < STEPS; ++s) {
    void* q1 = dev_fill(n1q);
    void* k1 = dev_fill(n1k);
    void* v1 = dev_fill(n1k);
    const int32_t h_pos[B] = {C + s, C + s};
    if (!q1 || !k1 || !v1 || !out1 || !lse1 || !pos ||
        hipMemcpy(pos, h_pos, sizeof h_pos, hipMemcpyHostToDevice) != hipSuccess) {
      fprintf(stderr, "decode inputs failed\n");
      return 1;
    }
    CHECK(swa_decode_step(&p, q1, k1, v1, kc, vc, pos, out1, (float*)lse1, dws, dws_bytes, 0));
    if (hipDeviceSynchronize() != hipSuccess || !dump(f, out1, n1q * 2) ||
        !dump(f, lse1, (size_t)B * HQ * 4)) {
      fprintf(stderr, "decode readback failed\n");
      return 1;
    }
    hipFree(q1);
    hipFree(k1);
    hipFree(v1);
  }
  if (!dump(f, kc, cache_bytes) || !dump(f, vc, cache_bytes)) {
    fprintf(stderr, "cache readback failed\n");
    return 1;
  }
  fclose(f);
  printf("swa_c_check: prefill %d tokens, %d decode steps, outputs in %s\n", C, STEPS, argv[1]);
  return 0;
}
