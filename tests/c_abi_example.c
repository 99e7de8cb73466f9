/*
 * The RFQ W4A4 linear layer through librfq's C ABI alone (include/rfq.h), as
 * a C program would use it: device buffers from hipMalloc, the weight
 * quantized once with rfq_quantize_mxfp4, the layer with rfq_linear and a
 * caller-owned workspace, every status checked. It also shows an argument
 * error coming back as a status with its detail text, with nothing launched.
 *
 * Inputs are fixed formulas whose values bfloat16 holds exactly:
 *   X[m][k] = ((131 m + 71 k) mod 97 - 48) / 16,  M x K
 *   W[n][k] = ((37 n + 53 k) mod 89 - 44) / 32,   N x K
 * Usage: c_abi_example OUT  -- writes Y (M x N float32, row-major) to OUT.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rfq.h"

enum { M = 300, N = 520, K = 1024 };

static uint16_t bf16_bits(float f) {   /* exact for the values above */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
  }
  return 0;
}

static int check_rfq(rfq_status_t st, const char* what) {
  if (st != RFQ_OK) {
    fprintf(stderr, "%s: %s (%s)\n", what, rfq_status_string(st), rfq_last_error_detail());
    return 1;
  }
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUT\n", argv[0]);
    return 2;
  }
  uint16_t* hx = malloc(sizeof(uint16_t) * M * K);
  uint16_t* hw = malloc(sizeof(uint16_t) * N * K);
  float* hy = malloc(sizeof(float) * M * N);
  if (!hx || !hw || !hy) return 3;
  for (int m = 0; m < M; ++m)
    for (int k = 0; k < K; ++k) hx[m * K + k] = bf16_bits((float)((131 * m + 71 * k) % 97 - 48) / 16.0f);
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) hw[n * K + k] = bf16_bits((float)((37 * n + 53 * k) % 89 - 44) / 32.0f);

  void *dx = NULL, *dw = NULL, *dy = NULL, *ws = NULL;
  uint8_t *wq = NULL, *sw = NULL;
  const size_t ws_bytes = rfq_linear_workspace_size(M, K);
  if (check_hip(hipMalloc(&dx, sizeof(uint16_t) * M * K), "hipMalloc x") ||
      check_hip(hipMalloc(&dw, sizeof(uint16_t) * N * K), "hipMalloc w") ||
      check_hip(hipMalloc(&dy, sizeof(float) * M * N), "hipMalloc y") ||
      check_hip(hipMalloc((void**)&wq, (size_t)N * K / 2), "hipMalloc wq") ||
      check_hip(hipMalloc((void**)&sw, (size_t)N * K / 32), "hipMalloc sw") ||
      check_hip(hipMalloc(&ws, ws_bytes), "hipMalloc workspace") ||
      check_hip(hipMemcpy(dx, hx, sizeof(uint16_t) * M * K, hipMemcpyHostToDevice), "copy x") ||
      check_hip(hipMemcpy(dw, hw, sizeof(uint16_t) * N * K, hipMemcpyHostToDevice), "copy w"))
    return 4;

  /* the weight, quantized once along K */
  if (check_rfq(rfq_quantize_mxfp4(dw, RFQ_DTYPE_BF16, N, K, K, wq, sw, NULL), "rfq_quantize_mxfp4")) return 5;

  /* an argument error: K not a multiple of 32 is rejected before any launch */
  rfq_status_t st = rfq_linear(dx, RFQ_DTYPE_BF16, M, 33, K, wq, sw, N, dy, RFQ_DTYPE_FP32, N, ws, ws_bytes, NULL);
  printf("K = 33: %s (%s)\n", rfq_status_string(st), rfq_last_error_detail());
  if (st != RFQ_ERR_INVALID_SHAPE) return 6;

  /* the layer: Q(X) and Q(R) into the workspace, then the K-doubled GEMM */
  if (check_rfq(rfq_linear(dx, RFQ_DTYPE_BF16, M, K, K, wq, sw, N, dy, RFQ_DTYPE_FP32, N, ws, ws_bytes, NULL),
                "rfq_linear"))
    return 7;
  if (check_hip(hipDeviceSynchronize(), "synchronize") ||
      check_hip(hipMemcpy(hy, dy, sizeof(float) * M * N, hipMemcpyDeviceToHost), "copy y"))
    return 8;

  FILE* f = fopen(argv[1], "wb");
  if (!f || fwrite(hy, sizeof(float), (size_t)M * N, f) != (size_t)M * N || fclose(f) != 0) return 9;
  printf("Y[0][0] = %g, Y[%d][%d] = %g\n", hy[0], M - 1, N - 1, hy[M * N - 1]);

  hipFree(dx);
  hipFree(dw);
  hipFree(dy);
  hipFree(wq);
  hipFree(sw);
  hipFree(ws);
  free(hx);
  free(hw);
  free(hy);
  return 0;
}
