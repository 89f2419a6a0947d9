/*
 * c_consumer.c -- a plain C program that uses libdsc through include/dsc.h
 * only: it allocates device memory with the HIP runtime, runs the head-wise
 * forward and backward and a low-rank forward, and writes the outputs to
 * files.  It shows that the library needs nothing from Python or PyTorch.
 *
 * usage: c_consumer <dir>
 *   reads  <dir>/in.bin  : int64 B, T, D, W, H, R then bf16 x (B,T,D),
 *                          w (B,T,D/H,W), dy (B,T,D), z (B,T,R), U (R,D*W)
 *   writes <dir>/out.bin : bf16 y, dx, dw (head-wise, residual) and
 *                          y (low-rank, H=1, SiLU)
 * Exit status 0 on success; any failing call prints dsc_last_error() and
 * exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dsc.h"

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));            \
      return 1;                                                             \
    }                                                                       \
  } while (0)

#define DSC_OK_(call)                                                       \
  do {                                                                      \
    dsc_status s_ = (call);                                                 \
    if (s_ != DSC_OK) {                                                     \
      fprintf(stderr, "%s: %s (%s)\n", #call, dsc_status_string(s_),        \
              dsc_last_error());                                            \
      return 1;                                                             \
    }                                                                       \
  } while (0)

static void *dev_copy(const void *host, size_t bytes) {
  void *p = NULL;
  if (hipMalloc(&p, bytes ? bytes : 16) != hipSuccess) return NULL;
  if (bytes && hipMemcpy(p, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return p;
}

int main(int argc, char **argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s <dir>\n", argv[0]);
    return 2;
  }
  char path[4096];
  snprintf(path, sizeof(path), "%s/in.bin", argv[1]);
  FILE *f = fopen(path, "rb");
  if (!f) { perror(path); return 1; }
  int64_t hdr[6];
  if (fread(hdr, sizeof(int64_t), 6, f) != 6) { fprintf(stderr, "short header\n"); return 1; }
  const int64_t B = hdr[0], T = hdr[1], D = hdr[2], W = hdr[3], H = hdr[4], R = hdr[5];
  const size_t n_act = (size_t)(B * T * D), n_w = (size_t)(B * T * (D / H) * W);
  const size_t n_z = (size_t)(B * T * R), n_u = (size_t)(R * D * W);
  const size_t n_in = 2 * n_act + n_w + n_z + n_u;
  uint16_t *in = (uint16_t *)malloc(n_in * 2);
  if (!in || fread(in, 2, n_in, f) != n_in) { fprintf(stderr, "short input\n"); return 1; }
  fclose(f);
  const uint16_t *hx = in, *hw = hx + n_act, *hdy = hw + n_w, *hz = hdy + n_act, *hU = hz + n_z;

  void *x = dev_copy(hx, n_act * 2), *w = dev_copy(hw, n_w * 2), *dy = dev_copy(hdy, n_act * 2);
  void *z = dev_copy(hz, n_z * 2), *U = dev_copy(hU, n_u * 2);
  void *y = NULL, *dx = NULL, *dw = NULL, *yl = NULL;
  if (!x || !w || !dy || !z || !U) { fprintf(stderr, "device copies failed\n"); return 1; }
  HIP_OK(hipMalloc(&y, n_act * 2));
  HIP_OK(hipMalloc(&dx, n_act * 2));
  HIP_OK(hipMalloc(&dw, n_w * 2));
  HIP_OK(hipMalloc(&yl, n_act * 2));
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));

  DSC_OK_(dsc_headwise_fwd(x, w, y, B, T, D, (int)W, (int)H, DSC_BF16, DSC_RESIDUAL, s));
  DSC_OK_(dsc_headwise_bwd(x, w, dy, dx, dw, B, T, D, (int)W, (int)H, DSC_BF16, DSC_RESIDUAL,
                           s));
  DSC_OK_(dsc_lowrank_fwd(x, z, U, yl, B, T, D, (int)W, 1, (int)R, DSC_BF16, DSC_ACT_SILU, s));
  /* a rejected call: H = 3 does not divide D */
  if (dsc_headwise_fwd(x, w, y, B, T, D, (int)W, 3, DSC_BF16, 0, s) == DSC_OK) {
    fprintf(stderr, "an invalid call was accepted\n");
    return 1;
  }
  HIP_OK(hipStreamSynchronize(s));

  uint16_t *out = (uint16_t *)malloc((3 * n_act + n_w) * 2);
  if (!out) return 1;
  HIP_OK(hipMemcpy(out, y, n_act * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out + n_act, dx, n_act * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out + 2 * n_act, dw, n_w * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out + 2 * n_act + n_w, yl, n_act * 2, hipMemcpyDeviceToHost));
  snprintf(path, sizeof(path), "%s/out.bin", argv[1]);
  f = fopen(path, "wb");
  if (!f || fwrite(out, 2, 3 * n_act + n_w, f) != 3 * n_act + n_w) { perror(path); return 1; }
  fclose(f);
  HIP_OK(hipStreamDestroy(s));
  hipFree(x); hipFree(w); hipFree(dy); hipFree(z); hipFree(U);
  hipFree(y); hipFree(dx); hipFree(dw); hipFree(yl);
  free(in);
  free(out);
  printf("c_consumer: ok (libdsc %d)\n", dsc_version());
  return 0;
}
