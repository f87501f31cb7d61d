/*
 * Host-side checks of the C ABI run under AddressSanitizer (built and run by
 * tests/test_host_asan.py against a copy of the library whose host code is
 * instrumented).  Every call here is answered on the host: queries that need
 * no device (status strings, sizes, plan names, the codebook) and entry
 * points whose arguments fail validation before anything is launched.  Host
 * buffers are heap blocks of exactly the size passed, so a write past the
 * size the caller gave is reported by the sanitizer.
 *
 * Prints "host asan ok" and returns 0 when every expectation holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "w4a16.h"

static int failures = 0;

#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                 \
    }                                                             \
  } while (0)

/* never dereferenced: every call below fails validation first */
static void* const FAKE = (void*)0x10000;
static void* const ODD = (void*)0x10008;

static void status_and_sizes(void) {
  for (int s = -3; s < 12; ++s) {
    const char* m = w4a16_status_string(s);
    EXPECT(m != NULL && strlen(m) > 0);
  }
  EXPECT(w4a16_version() >= 2);
  EXPECT(w4a16_repacked_bytes(4096, 4096, 128, 0) == 4096LL * 4096 / 2);
  EXPECT(w4a16_repacked_bytes(500, 256, 128, 0) == -1);
  EXPECT(w4a16_repacked_bytes(512, 20, 128, 0) == -1);
  EXPECT(w4a16_repacked_bytes(512, 256, 96, 0) == -1);
  EXPECT(w4a16_repacked_bytes(512, 256, 128, 7) == -1);
  for (int bits = 0; bits < 17; ++bits) {
    const int64_t r = w4a16_repacked_bytes_bits(4096, 4096, 128, bits, 0);
    EXPECT((bits == 3 || bits == 4 || bits == 8) ? r == 4096LL * 4096 * bits / 8 : r == -1);
  }
  EXPECT(w4a16_workspace_bytes(1, 4096, 4096, 128) == 0);
  EXPECT(w4a16_workspace_bytes(16, 4096, 4096, 128) >= 16 * 4096 * 2);
  EXPECT(w4a16_workspace_bytes(0, 4096, 4096, 128) == -1);
  EXPECT(w4a16_workspace_bytes((int64_t)1 << 20, 256, (int64_t)1 << 17, 128) == -1);
  EXPECT(nf4_workspace_bytes(1, 28672, 8192, 64) == 0);
  EXPECT(nf4_workspace_bytes(1, 28672, 8192, 32) == -1);
}

/* every buffer size from 0 to past the full name: the library must write at
 * most `size` bytes, NUL-terminated, and report the full length */
static void plan_names(void) {
  static const int64_t shapes[][3] = {{1, 4096, 4096},   {4, 11008, 4096}, {16, 4096, 11008},
                                      {24, 4096, 4096},  {64, 5120, 5120}, {2048, 5120, 7168},
                                      {2100, 55296, 5120}, {4, 1024, 98304}};
  for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
    for (int perm = 0; perm < 2; ++perm) {
      int64_t full = -1;
      EXPECT(w4a16_gemm_plan(shapes[i][0], shapes[i][1], shapes[i][2], 128, 4, 0, perm, 0, 1,
                             NULL, 0, &full) == 0);
      EXPECT(full > 8);
      for (int64_t n = 1; n <= full + 2; ++n) {
        char* b = (char*)malloc((size_t)n);
        int64_t len = -1;
        EXPECT(w4a16_gemm_plan(shapes[i][0], shapes[i][1], shapes[i][2], 128, 4, 0, perm, 0, 1,
                               b, n, &len) == 0);
        EXPECT(len == full);
        EXPECT((int64_t)strlen(b) == (n - 1 < full ? n - 1 : full));
        free(b);
      }
    }
  }
  for (int64_t M = 1; M <= 64; M += 31) {
    int64_t full = -1;
    EXPECT(nf4_gemm_plan(M, 28672, 8192, 64, 1, 1, NULL, 0, &full) == 0);
    for (int64_t n = 1; n <= full + 2; ++n) {
      char* b = (char*)malloc((size_t)n);
      EXPECT(nf4_gemm_plan(M, 28672, 8192, 64, 1, 1, b, n, NULL) == 0);
      EXPECT((int64_t)strlen(b) == (n - 1 < full ? n - 1 : full));
      free(b);
    }
  }
  for (int64_t M = 1; M <= 2048; M *= 8) {
    int64_t full = -1;
    EXPECT(nf4_gemm_repacked_plan(M, 28672, 8192, 64, 1, 1, NULL, 0, &full) == 0);
    for (int64_t n = 1; n <= full + 2; ++n) {
      char* b = (char*)malloc((size_t)n);
      EXPECT(nf4_gemm_repacked_plan(M, 28672, 8192, 64, 1, 1, b, n, NULL) == 0);
      EXPECT((int64_t)strlen(b) == (n - 1 < full ? n - 1 : full));
      free(b);
    }
  }
  EXPECT(nf4_gemm_plan(1, 28672, 8192, 64, 1, 1, NULL, 8, NULL) == W4A16_ERR_INVALID_ARG);
  EXPECT(w4a16_gemm_plan(0, 256, 512, 128, 4, 0, 0, 0, 1, NULL, 0, NULL) ==
         W4A16_ERR_INVALID_ARG);
}

static void codebook(void) {
  float* L = (float*)malloc(16 * sizeof(float));
  EXPECT(nf4_codebook(L) == 0);
  EXPECT(L[0] == -1.0f && L[7] == 0.0f && L[15] == 1.0f);
  free(L);
  EXPECT(nf4_codebook(NULL) != 0);
}

static void validation(void) {
  /* w4a16_gemm: M <= 0, K % G, unsupported G, dtype, NULL, misaligned, workspace */
  EXPECT(w4a16_gemm(FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 0, 256, 512, 0, NULL, 0, NULL) == 1);
  EXPECT(w4a16_gemm(FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 1, 256, 500, 0, NULL, 0, NULL) == 1);
  EXPECT(w4a16_gemm(FAKE, FAKE, FAKE, FAKE, NULL, 96, FAKE, 1, 256, 512, 0, NULL, 0, NULL) == 2);
  EXPECT(w4a16_gemm(FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 1, 256, 512, 7, NULL, 0, NULL) == 1);
  EXPECT(w4a16_gemm(NULL, FAKE, FAKE, FAKE, NULL, 128, FAKE, 1, 256, 512, 0, NULL, 0, NULL) == 1);
  EXPECT(w4a16_gemm(ODD, FAKE, FAKE, FAKE, NULL, 128, FAKE, 1, 256, 512, 0, NULL, 0, NULL) == 3);
  const int64_t need = w4a16_workspace_bytes(16, 4096, 4096, 128);
  EXPECT(w4a16_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, 16, 4096, 4096, 0, FAKE, need - 16,
                    NULL) == 5);
  EXPECT(w4a16_gemm_xscale(FAKE, ODD, FAKE, FAKE, FAKE, NULL, 128, FAKE, 2, 4096, 4096, 0, NULL,
                           0, NULL) == 3);
  EXPECT(w4a16_gemm_bits(FAKE, NULL, FAKE, FAKE, FAKE, NULL, 128, 6, FAKE, 1, 256, 512, 0, NULL,
                         0, NULL) == 2);
  EXPECT(w4a16_gemm_noalloc(FAKE, NULL, FAKE, FAKE, FAKE, NULL, 128, 4, FAKE, 0, 256, 512, 0,
                            NULL) == 1);
  EXPECT(w4a16_dequant_bits(FAKE, FAKE, FAKE, 512, 256, 128, 7, 0, FAKE, NULL) == 2);
  /* repack / quantize */
  int32_t used = 0;
  EXPECT(w4a16_repack(FAKE, FAKE, FAKE, FAKE, 512, 256, 128, FAKE, FAKE, FAKE, NULL, &used,
                      NULL) == 1);
  EXPECT(w4a16_repack(FAKE, FAKE, NULL, NULL, 512, 256, 96, FAKE, FAKE, NULL, NULL, &used,
                      NULL) == 2);
  EXPECT(w4a16_repack_bits(FAKE, FAKE, FAKE, NULL, 512, 200, 128, 3, FAKE, FAKE, FAKE, NULL,
                           &used, NULL) == 1);
  EXPECT(w4a16_quantize_rtn(FAKE, FAKE, NULL, 256, 512, 128, FAKE, FAKE, FAKE, NULL) == 1);
  EXPECT(w4a16_quantize_rtn_bits(FAKE, NULL, NULL, 256, 512, 128, 2, FAKE, FAKE, FAKE, NULL) ==
         2);
  /* NF4 */
  EXPECT(nf4_gemm(FAKE, FAKE, FAKE, FAKE, 32, FAKE, 1, 256, 512, 1, NULL, 0, NULL) == 2);
  EXPECT(nf4_gemm(FAKE, FAKE, FAKE, FAKE, 64, FAKE, 1, 256, 96, 1, NULL, 0, NULL) == 1);
  EXPECT(nf4_gemm(FAKE, NULL, FAKE, FAKE, 64, FAKE, 1, 256, 512, 1, NULL, 0, NULL) == 1);
  EXPECT(nf4_quantize(FAKE, 16, 100, 64, FAKE, FAKE, FAKE, NULL) == 1);
  EXPECT(nf4_repacked_bytes(16, 320, 64) == 3 * 1024);
  EXPECT(nf4_repacked_bytes(20, 320, 64) == -1);
  EXPECT(nf4_repack(FAKE, 20, 320, 64, FAKE, NULL) == 1);
  EXPECT(nf4_gemm_repacked(FAKE, FAKE, FAKE, FAKE, 32, FAKE, 1, 256, 512, 1, NULL, 0, NULL) ==
         2);
  EXPECT(w4a16_set_timing_events(NULL, NULL) == 0);
}

int main(void) {
  status_and_sizes();
  plan_names();
  codebook();
  validation();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host asan ok\n");
  return 0;
}
