/*
 * A C program that drives libfp8mi through its C ABI alone: the HIP runtime
 * for device memory and copies, include/fp8mi.h for every call -- no Python,
 * no torch.  tests/test_c_abi_gpu.py compiles it with gcc, feeds it inputs
 * and checks its outputs against the oracle.
 *
 *   c_abi_demo IN OUT
 *
 * IN  (little-endian): int64 rows, int64 cols, int64 n, float32 s0 (the
 *     x ring's starting scale), float32 sw (W's explicit scale), then the
 *     bf16 bit patterns of X [rows, cols] and W [n, cols].
 * Steps: X -> E4M3 row codes with a 4-entry ring (fold in-kernel); W -> E4M3
 *     codes in both layouts at scale sw; Y = Xq Wq^T (bf16, scale_inv of both);
 *     one more fold of X's amax through fp8_amax_fold; one rejected call.
 * OUT: int32 status of the rejected call, int32 length of its error text,
 *     float32 sx, ax, sw_inv, aw, the ring's 4 + 4 + 1024 words, then the codes
 *     Xq [rows, cols], Wq [n, cols], WqT [cols, n] and Y [rows, n] (bf16 bits).
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8mi.h"

#define H 4

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static int lib_ok(fp8mi_status s, const char* what) {
  if (s != FP8MI_OK) {
    fprintf(stderr, "%s: %s -- %s\n", what, fp8mi_status_string(s), fp8mi_last_error());
    return 0;
  }
  return 1;
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  return hip_ok(hipMalloc(&p, bytes ? bytes : 1), "hipMalloc") ? p : NULL;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 2;
  int64_t rows, cols, n;
  float s0, sw;
  if (fread(&rows, 8, 1, in) != 1 || fread(&cols, 8, 1, in) != 1 || fread(&n, 8, 1, in) != 1 ||
      fread(&s0, 4, 1, in) != 1 || fread(&sw, 4, 1, in) != 1)
    return 2;
  if (rows < 1 || cols < 1 || n < 1 || rows > 4096 || cols > 4096 || n > 4096) return 2;
  const size_t nx = (size_t)(rows * cols), nw = (size_t)(n * cols), ny = (size_t)(rows * n);
  uint16_t* hx = malloc(2 * nx);
  uint16_t* hw = malloc(2 * nw);
  if (!hx || !hw || fread(hx, 2, nx, in) != nx || fread(hw, 2, nw, in) != nw) return 2;
  fclose(in);

  const size_t ring_words = FP8MI_RING_WORDS(H);
  uint32_t* hring = calloc(ring_words, 4);
  memcpy(&hring[H], &s0, 4);  /* history 0, slot 0, scale s0, everything else 0 */

  uint16_t *dx = dev_alloc(2 * nx), *dw = dev_alloc(2 * nw), *dy = dev_alloc(2 * ny);
  uint8_t *xq = dev_alloc(nx), *wq = dev_alloc(nw), *wqt = dev_alloc(nw);
  uint32_t* ring = dev_alloc(4 * ring_words);
  float* scal = dev_alloc(5 * sizeof(float)); /* sx, ax, sw_inv, aw, sw */
  if (!dx || !dw || !dy || !xq || !wq || !wqt || !ring || !scal) return 3;
  if (!hip_ok(hipMemcpy(dx, hx, 2 * nx, hipMemcpyHostToDevice), "copy x") ||
      !hip_ok(hipMemcpy(dw, hw, 2 * nw, hipMemcpyHostToDevice), "copy w") ||
      !hip_ok(hipMemcpy(ring, hring, 4 * ring_words, hipMemcpyHostToDevice), "copy ring") ||
      !hip_ok(hipMemcpy(scal + 4, &sw, 4, hipMemcpyHostToDevice), "copy sw"))
    return 3;

  /* every call on the null stream, in order */
  if (!lib_ok(fp8_quantize(dx, FP8MI_BF16, rows, cols, cols, FP8MI_E4M3, 0, xq, cols, NULL, ring, H, scal + 0,
                           scal + 1, NULL), "fp8_quantize") ||
      !lib_ok(fp8_quantize_dual(dw, FP8MI_BF16, n, cols, cols, FP8MI_E4M3, wq, cols, wqt, n, scal + 4, NULL, 0,
                                scal + 2, scal + 3, NULL), "fp8_quantize_dual") ||
      !lib_ok(fp8_mm(xq, FP8MI_E4M3, cols, 0, wq, FP8MI_E4M3, cols, 0, rows, n, cols, 1, scal + 0, scal + 2, NULL,
                     FP8MI_BF16, dy, n, 0, NULL), "fp8_mm") ||
      !lib_ok(fp8_amax_fold(ring, H, scal + 1, FP8MI_E4M3, NULL), "fp8_amax_fold"))
    return 4;
  /* a rejected call: an unknown format, refused before anything is launched */
  const int32_t bad = (int32_t)fp8_quantize(dx, FP8MI_BF16, rows, cols, cols, 7, 0, xq, cols, NULL, ring, H, NULL,
                                            NULL, NULL);
  const int32_t bad_len = (int32_t)strlen(fp8mi_last_error());
  if (!hip_ok(hipDeviceSynchronize(), "synchronize")) return 5;

  float hs[4];
  uint8_t* hq = malloc(nx + 2 * nw);
  uint16_t* hy = malloc(2 * ny);
  if (!hq || !hy || !hip_ok(hipMemcpy(hs, scal, 16, hipMemcpyDeviceToHost), "copy scalars") ||
      !hip_ok(hipMemcpy(hring, ring, 4 * ring_words, hipMemcpyDeviceToHost), "copy ring") ||
      !hip_ok(hipMemcpy(hq, xq, nx, hipMemcpyDeviceToHost), "copy xq") ||
      !hip_ok(hipMemcpy(hq + nx, wq, nw, hipMemcpyDeviceToHost), "copy wq") ||
      !hip_ok(hipMemcpy(hq + nx + nw, wqt, nw, hipMemcpyDeviceToHost), "copy wqt") ||
      !hip_ok(hipMemcpy(hy, dy, 2 * ny, hipMemcpyDeviceToHost), "copy y"))
    return 5;

  FILE* out = fopen(argv[2], "wb");
  if (!out) return 6;
  fwrite(&bad, 4, 1, out);
  fwrite(&bad_len, 4, 1, out);
  fwrite(hs, 4, 4, out);
  fwrite(hring, 4, ring_words, out);
  fwrite(hq, 1, nx + 2 * nw, out);
  fwrite(hy, 2, ny, out);
  fclose(out);

  hipFree(dx); hipFree(dw); hipFree(dy); hipFree(xq); hipFree(wq); hipFree(wqt); hipFree(ring); hipFree(scal);
  free(hx); free(hw); free(hring); free(hq); free(hy);
  printf("c_abi_demo ok: %s\n", fp8mi_version());
  return 0;
}
