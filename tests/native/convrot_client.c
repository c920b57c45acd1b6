/*
 * convrot_client.c -- a plain C99 client of libconvrot: the ConvLinear4bit forward pass
 * driven through include/convrot.h and the HIP runtime's C API alone.  No C++, Python or
 * torch runs in this process; the tests use it to show that the C ABI stands on its own.
 *
 * Usage:
 *   convrot_client forward X W BIAS M K N G OUT
 *       X: bf16 [M][K], W: bf16 [N][K], BIAS: bf16 [N] or "-" for none, all raw
 *       little-endian files; OUT receives y bf16 [M][N].  Steps: offline weight codes
 *       (convrot_quant_weight), workspace sizing and allocation (convrot_w4a4_workspace_bytes),
 *       the forward pass (convrot_w4a4_linear) on a stream of its own, y copied back.
 *   convrot_client errors
 *       Host validation only (no device memory, no launch): invalid arguments come back as
 *       the status codes include/convrot.h documents.
 * Exit status 0 on success; otherwise a message on stderr names the failing call.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "convrot.h"

static int fail(const char* what, int st) {
  fprintf(stderr, "convrot_client: %s: %d (%s)\n", what, st, convrot_status_string(st));
  return 1;
}

#define HIP_OK(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "convrot_client: %s: %s\n", #call, hipGetErrorString(e_));      \
      return 1;                                                                       \
    }                                                                                 \
  } while (0)

static void* read_file(const char* path, size_t bytes) {
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* buf = malloc(bytes ? bytes : 1);
  size_t got = buf ? fread(buf, 1, bytes, f) : 0;
  int extra = fgetc(f) != EOF;  /* the file must hold exactly `bytes` */
  fclose(f);
  if (!buf || got != bytes || extra) {
    free(buf);
    return NULL;
  }
  return buf;
}

/* Every check here fails validation before any device work, so it needs no GPU. */
static int check_errors(void) {
  /* Distinct non-NULL addresses that are never dereferenced: validation rejects each call
   * before any launch. */
  static uint8_t dummy[4096] __attribute__((aligned(256)));
  void* p = dummy;
  struct {
    const char* what;
    int got, want;
  } cases[] = {
      {"padded_k(100, 8)", (int)convrot_padded_k(100, 8), CONVROT_ERR_GROUP},
      {"padded_k(0, 16)", (int)convrot_padded_k(0, 16), CONVROT_ERR_SHAPE},
      {"padded_k(3100, 256) = 3328", (int)convrot_padded_k(3100, 256), 3328},
      {"is_power_of_4(1024)", convrot_is_power_of_4(1024), 1},
      {"is_power_of_4(32)", convrot_is_power_of_4(32), 0},
      {"linear, g = 8",
       convrot_w4a4_linear(p, CONVROT_BF16, 4, 64, 8, dummy, (float*)p, 4, NULL, p, p, 4096, NULL),
       CONVROT_ERR_GROUP},
      {"linear, g = 4096",
       convrot_w4a4_linear(p, CONVROT_BF16, 4, 64, 4096, dummy, (float*)p, 4, NULL, p, p, 4096, NULL),
       CONVROT_ERR_UNSUPPORTED},
      {"linear, x = NULL",
       convrot_w4a4_linear(NULL, CONVROT_BF16, 4, 64, 16, dummy, (float*)p, 4, NULL, p, p, 4096, NULL),
       CONVROT_ERR_NULL},
      {"linear, dtype 7",
       convrot_w4a4_linear(p, 7, 4, 64, 16, dummy, (float*)p, 4, NULL, p, p, 4096, NULL),
       CONVROT_ERR_DTYPE},
      {"linear, M < 0",
       convrot_w4a4_linear(p, CONVROT_BF16, -1, 64, 16, dummy, (float*)p, 4, NULL, p, p, 4096, NULL),
       CONVROT_ERR_SHAPE},
      {"linear, workspace too small",
       convrot_w4a4_linear(p, CONVROT_BF16, 4, 64, 16, dummy, (float*)p, 4, NULL, p, p, 16, NULL),
       CONVROT_ERR_WORKSPACE},
      {"workspace_bytes(4, 64, 8) = 0", (int)convrot_w4a4_workspace_bytes(4, 64, 8), 0},
      {"rotate_quant, xq misaligned",
       convrot_rotate_quant_act(p, CONVROT_BF16, 4, 64, 64, 16, dummy + 1, (float*)p, NULL, NULL),
       CONVROT_ERR_ALIGN},
      {"gemm, Kp = 40",
       convrot_w4a4_gemm(dummy, (float*)p, dummy, (float*)p, NULL, 4, 4, 40, p, NULL, NULL),
       CONVROT_ERR_SHAPE},
  };
  int bad = 0;
  for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i) {
    if (cases[i].got != cases[i].want) {
      fprintf(stderr, "convrot_client: %s returned %d (%s), expected %d\n", cases[i].what,
              cases[i].got, convrot_status_string(cases[i].got), cases[i].want);
      bad = 1;
    }
  }
  if (!bad) printf("convrot_client: %zu validation checks ok (library %d)\n",
                   sizeof(cases) / sizeof(cases[0]), convrot_version());
  return bad;
}

static int forward(char** a) {
  const int64_t M = atoll(a[3]), K = atoll(a[4]), N = atoll(a[5]), g = atoll(a[6]);
  const int64_t Kp = convrot_padded_k(K, g);
  if (M < 1 || N < 1 || Kp < 0) return fail("shape", Kp < 0 ? (int)Kp : CONVROT_ERR_SHAPE);
  const size_t xb = (size_t)(M * K * 2), wb = (size_t)(N * K * 2), bb = (size_t)(N * 2);
  const size_t yb = (size_t)(M * N * 2);
  void* hx = read_file(a[0], xb);
  void* hw = read_file(a[1], wb);
  void* hb = strcmp(a[2], "-") ? read_file(a[2], bb) : NULL;
  if (!hx || !hw || (strcmp(a[2], "-") && !hb)) {
    fprintf(stderr, "convrot_client: an input file is missing or has the wrong size\n");
    return 1;
  }
  const size_t ws_bytes = convrot_w4a4_workspace_bytes(M, K, g);
  if (ws_bytes == 0) return fail("convrot_w4a4_workspace_bytes", CONVROT_ERR_SHAPE);

  hipStream_t stream;
  void *dx, *dw, *db = NULL, *dy, *dwq, *dws, *dwork;
  HIP_OK(hipStreamCreate(&stream));
  HIP_OK(hipMalloc(&dx, xb));
  HIP_OK(hipMalloc(&dw, wb));
  HIP_OK(hipMalloc(&dy, yb));
  HIP_OK(hipMalloc(&dwq, (size_t)(N * Kp / 2)));
  HIP_OK(hipMalloc(&dws, (size_t)(N * 4)));
  HIP_OK(hipMalloc(&dwork, ws_bytes));
  HIP_OK(hipMemcpy(dx, hx, xb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dw, hw, wb, hipMemcpyHostToDevice));
  if (hb) {
    HIP_OK(hipMalloc(&db, bb));
    HIP_OK(hipMemcpy(db, hb, bb, hipMemcpyHostToDevice));
  }

  int st = convrot_quant_weight(dw, CONVROT_BF16, N, K, g, (uint8_t*)dwq, (float*)dws, stream);
  if (st != CONVROT_OK) return fail("convrot_quant_weight", st);
  st = convrot_w4a4_linear(dx, CONVROT_BF16, M, K, g, (const uint8_t*)dwq, (const float*)dws, N,
                           db, dy, dwork, ws_bytes, stream);
  if (st != CONVROT_OK) return fail("convrot_w4a4_linear", st);
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipGetLastError());

  void* hy = malloc(yb);
  if (!hy) return 1;
  HIP_OK(hipMemcpy(hy, dy, yb, hipMemcpyDeviceToHost));
  FILE* f = fopen(a[7], "wb");
  if (!f || fwrite(hy, 1, yb, f) != yb || fclose(f) != 0) {
    fprintf(stderr, "convrot_client: cannot write %s\n", a[7]);
    return 1;
  }
  HIP_OK(hipFree(dx));
  HIP_OK(hipFree(dw));
  HIP_OK(hipFree(dy));
  HIP_OK(hipFree(dwq));
  HIP_OK(hipFree(dws));
  HIP_OK(hipFree(dwork));
  if (db) HIP_OK(hipFree(db));
  HIP_OK(hipStreamDestroy(stream));
  free(hx);
  free(hw);
  free(hb);
  free(hy);
  printf("convrot_client: forward M=%lld K=%lld N=%lld g=%lld ok\n", (long long)M, (long long)K,
         (long long)N, (long long)g);
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "errors") == 0) return check_errors();
  if (argc == 10 && strcmp(argv[1], "forward") == 0) return forward(argv + 2);
  fprintf(stderr,
          "usage: convrot_client forward X W BIAS|- M K N G OUT\n"
          "       convrot_client errors\n");
  return 2;
}
