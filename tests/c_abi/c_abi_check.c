/*
 * A plain C program that uses librar.so through include/rar.h alone, with
 * device memory from the HIP runtime API: no Python, no torch.  It checks
 * that the boundary is usable from C.
 *
 *   c_abi_check --cpu   host-only calls (sizes, plans, argument errors)
 *   c_abi_check         the above, then on the GPU: fused and stepwise ring
 *                       allreduce, BFP-8 compressed ring and tree allreduce
 *                       of integer-valued fp32/fp16 inputs, whose sums are
 *                       exact in any order, compared with the exact sum.
 *
 * Prints "c_abi_check OK" and exits 0 on success; names the failing check
 * and exits 1 otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rar.h"

static int failures = 0;

#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) {                                \
      fprintf(stderr, "FAILED: " __VA_ARGS__);    \
      fprintf(stderr, "  (%s:%d)\n", __FILE__, __LINE__); \
      ++failures;                                 \
    }                                             \
  } while (0)

/* x_r[i] = ((5 i + 3 r) mod 13) - 6: small integers, exact in fp16 and fp32 */
static float value(size_t i, int r) { return (float)((int)((5 * i + 3 * (size_t)r) % 13) - 6); }

static uint16_t f32_to_f16_int(float f) {
  /* integers |v| <= 2048 only: sign, exponent, 10-bit fraction, exact */
  if (f == 0.0f) return 0;
  uint16_t s = f < 0 ? 0x8000 : 0;
  float a = fabsf(f);
  int e = 0;
  while (a >= 2.0f) { a /= 2.0f; ++e; }
  uint16_t frac = (uint16_t)((a - 1.0f) * 1024.0f);
  return (uint16_t)(s | (uint16_t)((e + 15) << 10) | frac);
}

static float f16_to_f32_int(uint16_t h) {
  if ((h & 0x7fff) == 0) return 0.0f;
  int e = ((h >> 10) & 0x1f) - 15;
  float v = (1.0f + (float)(h & 0x3ff) / 1024.0f) * ldexpf(1.0f, e);
  return (h & 0x8000) ? -v : v;
}

static void host_checks(void) {
  CHECK(strstr(rar_version(), "gfx950") != NULL, "version string\n");
  CHECK(strcmp(rar_status_string(RAR_OK), "ok") == 0, "status string\n");
  CHECK(rar_chunk_len(1000, 3) == 384, "chunk_len(1000, 3)\n");
  CHECK(rar_chunk_len(64u << 20, 8) == (8u << 20), "chunk_len(64M, 8)\n");
  CHECK(rar_bfp_bytes(128 * 37 + 5, 128, 8) == 48 + 128 * 37 + 5, "bfp_bytes m=8\n");
  CHECK(rar_bfp_bytes(256, 128, 4) == 16 + 128, "bfp_bytes m=4\n");
  size_t counts[6] = {10, 20, 5, 100, 3, 3};
  int plan[6];
  CHECK(rar_bucket_plan(counts, 6, RAR_BF16, 60, plan) == 4, "bucket plan count\n");
  CHECK(plan[0] == 0 && plan[1] == 0 && plan[2] == 1 && plan[3] == 2 && plan[4] == 3 && plan[5] == 3,
        "bucket plan\n");
  rar_compress_cfg cfg;
  rar_compress_cfg_default(&cfg);
  CHECK(cfg.method == RAR_COMP_BFP && cfg.block == 128 && cfg.mbits == 8, "default compression config\n");
  /* argument errors come back before anything touches the device */
  void* fake[2] = {(void*)(uintptr_t)(1ull << 40), (void*)(uintptr_t)((1ull << 40) + 16)};
  CHECK(rar_ring_allreduce(fake, 2, 1024, RAR_F32, NULL) == RAR_EOVERLAP, "overlap detected\n");
  CHECK(rar_ring_allreduce(fake, 2, 1024, 9, NULL) == RAR_EDTYPE, "dtype rejected\n");
  CHECK(rar_ring_allreduce(fake, 0, 1024, RAR_F32, NULL) == RAR_EINVAL, "rank count rejected\n");
  CHECK(rar_ring_allreduce(fake, 2, 0, RAR_F32, NULL) == RAR_OK, "empty allreduce is a no-op\n");
}

static int dev_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "FAILED: %s: %s\n", what, hipGetErrorString(e));
    ++failures;
    return 0;
  }
  return 1;
}

/* n rank buffers of count elements of dtype (F32 or F16), integer inputs */
static int run_case(int n, size_t count, int dtype, const char* what,
                    int (*op)(void* const*, int, size_t, int, void*, void*), void* ctx) {
  const size_t es = dtype == RAR_F32 ? 4 : 2, bytes = count * es;
  void* bufs[RAR_MAX_RANKS];
  unsigned char* host = (unsigned char*)malloc(bytes);
  for (int r = 0; r < n; ++r) {
    if (!dev_ok(hipMalloc(&bufs[r], bytes), "hipMalloc")) return 0;
    for (size_t i = 0; i < count; ++i) {
      float v = value(i, r);
      if (dtype == RAR_F32) memcpy(host + 4 * i, &v, 4);
      else { uint16_t h = f32_to_f16_int(v); memcpy(host + 2 * i, &h, 2); }
    }
    if (!dev_ok(hipMemcpy(bufs[r], host, bytes, hipMemcpyHostToDevice), "upload")) return 0;
  }
  int rc = op(bufs, n, count, dtype, NULL, ctx);
  CHECK(rc == RAR_OK, "%s returned %d (%s)\n", what, rc, rar_status_string(rc));
  dev_ok(hipDeviceSynchronize(), "synchronize");
  for (int r = 0; r < n && rc == RAR_OK; ++r) {
    if (!dev_ok(hipMemcpy(host, bufs[r], bytes, hipMemcpyDeviceToHost), "download")) break;
    for (size_t i = 0; i < count; ++i) {
      float want = 0.0f, got;
      for (int q = 0; q < n; ++q) want += value(i, q);
      if (dtype == RAR_F32) memcpy(&got, host + 4 * i, 4);
      else { uint16_t h; memcpy(&h, host + 2 * i, 2); got = f16_to_f32_int(h); }
      if (got != want) {
        fprintf(stderr, "FAILED: %s rank %d element %zu: %g != %g\n", what, r, i, got, want);
        ++failures;
        break;
      }
    }
  }
  for (int r = 0; r < n; ++r) hipFree(bufs[r]);
  free(host);
  return rc == RAR_OK;
}

static int op_fused(void* const* b, int n, size_t c, int dt, void* s, void* ctx) {
  (void)ctx;
  return rar_ring_allreduce_ex(b, n, c, dt, RAR_ALGO_FUSED, s);
}
static int op_stepwise(void* const* b, int n, size_t c, int dt, void* s, void* ctx) {
  (void)ctx;
  return rar_ring_allreduce_ex(b, n, c, dt, RAR_ALGO_STEPWISE, s);
}
static int op_tree(void* const* b, int n, size_t c, int dt, void* s, void* ctx) {
  (void)ctx;
  return rar_tree_allreduce(b, n, c, dt, s);
}
static int op_bfp(void* const* b, int n, size_t c, int dt, void* s, void* ctx) {
  rar_compress_cfg cfg;
  rar_compress_cfg_default(&cfg);
  cfg.schedule = *(const int*)ctx;
  cfg.unit_bytes = 64 << 10;
  size_t ws_bytes = rar_compressed_workspace_bytes(n, c, dt, &cfg);
  void* ws = NULL;
  if (hipMalloc(&ws, ws_bytes) != hipSuccess) return RAR_EHIP;
  int rc = rar_ring_allreduce_compressed(b, n, c, dt, &cfg, ws, ws_bytes, s);
  if (rc == RAR_OK) {
    uint64_t sent[RAR_MAX_RANKS], recv[RAR_MAX_RANKS];
    rc = rar_compressed_traffic(ws, n, sent, recv, s);
  }
  hipDeviceSynchronize();
  hipFree(ws);
  return rc;
}

int main(int argc, char** argv) {
  host_checks();
  if (argc > 1 && strcmp(argv[1], "--cpu") == 0) {
    if (failures) return 1;
    printf("c_abi_check OK (host calls)\n");
    return 0;
  }
  int ndev = 0;
  if (!dev_ok(hipGetDeviceCount(&ndev), "hipGetDeviceCount") || ndev < 1) return 1;
  const size_t count = 3 * 4096 + 1001;
  run_case(8, count, RAR_F32, "fused fp32 allreduce", op_fused, NULL);
  run_case(5, count, RAR_F16, "stepwise fp16 allreduce", op_stepwise, NULL);
  run_case(4, count, RAR_F32, "tree fp32 allreduce", op_tree, NULL);
  int scheds[4] = {RAR_SCHED_FUSED, RAR_SCHED_STAGED, RAR_SCHED_FORWARD, RAR_SCHED_PIPELINED};
  const char* names[4] = {"BFP-8 fused", "BFP-8 staged", "BFP-8 forward", "BFP-8 pipelined"};
  for (int k = 0; k < 4; ++k) run_case(4, 64 * 1024 + 300, RAR_F16, names[k], op_bfp, &scheds[k]);
  if (failures) return 1;
  printf("c_abi_check OK\n");
  return 0;
}
