/* A plain C99 client of include/cce.h: libcce without Python or PyTorch.
 *
 * Reads a problem from IN (a header of int64 N, V, D, ignore_index and float filter_eps, then
 * E [N][D] and C [V][D] as bf16 bit patterns (uint16), targets [N] int64 and dloss [N] float),
 * allocates every device buffer with the HIP runtime's C API, queries the workspace sizes,
 * runs cce_forward (with the tile maxima) and cce_backward (fp32 gradients, skip statistics)
 * on one stream, and writes loss [N], lse [N], dE [N][D], dC [V][D] (float) and the two skip
 * counts (int64) to OUT.  Exit status 0 on success; any library or runtime error is printed
 * with its name and gives status 1.
 *
 * usage: cce_c_client IN OUT */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "cce.h"

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

#define CCE_OK_(call)                                                             \
  do {                                                                            \
    cce_status s_ = (call);                                                       \
    if (s_ != CCE_OK) {                                                           \
      fprintf(stderr, "%s failed: %s\n", #call, cce_status_string(s_));           \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

static int read_all(FILE* f, void* dst, size_t bytes) {
  return fread(dst, 1, bytes, f) == bytes;
}

static int write_all(FILE* f, const void* src, size_t bytes) {
  return fwrite(src, 1, bytes, f) == bytes;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 1;
  }
  int64_t hdr[4];
  float eps;
  if (!read_all(in, hdr, sizeof hdr) || !read_all(in, &eps, sizeof eps)) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int64_t N = hdr[0], V = hdr[1], D = hdr[2], ii = hdr[3];
  if (N < 1 || V < 1 || D < 1) {
    fprintf(stderr, "bad sizes\n");
    return 1;
  }
  const size_t nE = (size_t)N * (size_t)D, nC = (size_t)V * (size_t)D;
  uint16_t* hE = malloc(nE * 2);
  uint16_t* hC = malloc(nC * 2);
  int64_t* ht = malloc((size_t)N * 8);
  float* hdl = malloc((size_t)N * 4);
  if (!hE || !hC || !ht || !hdl || !read_all(in, hE, nE * 2) || !read_all(in, hC, nC * 2) ||
      !read_all(in, ht, (size_t)N * 8) || !read_all(in, hdl, (size_t)N * 4)) {
    fprintf(stderr, "short input\n");
    return 1;
  }
  fclose(in);

  const size_t fws = cce_forward_workspace_bytes(N, V, D, CCE_BF16);
  const size_t bws = cce_backward_workspace_bytes(N, V, D, CCE_BF16, CCE_F32);
  const int64_t ntm = cce_tile_max_count(N, V, D, CCE_BF16);
  if (fws == 0 || bws == 0 || ntm <= 0) {
    fprintf(stderr, "the workspace queries refused the sizes\n");
    return 1;
  }

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  void *dEin, *dCin, *dws_f, *dws_b, *ddE, *ddC;
  int64_t *dt, *dstats;
  float *ddl, *dloss, *dlse, *dtm;
  HIP_OK(hipMalloc(&dEin, nE * 2));
  HIP_OK(hipMalloc(&dCin, nC * 2));
  HIP_OK(hipMalloc((void**)&dt, (size_t)N * 8));
  HIP_OK(hipMalloc((void**)&ddl, (size_t)N * 4));
  HIP_OK(hipMalloc((void**)&dloss, (size_t)N * 4));
  HIP_OK(hipMalloc((void**)&dlse, (size_t)N * 4));
  HIP_OK(hipMalloc((void**)&dtm, (size_t)ntm * 4));
  HIP_OK(hipMalloc(&dws_f, fws));
  HIP_OK(hipMalloc(&dws_b, bws));
  HIP_OK(hipMalloc(&ddE, nE * 4));
  HIP_OK(hipMalloc(&ddC, nC * 4));
  HIP_OK(hipMalloc((void**)&dstats, 2 * 8));
  HIP_OK(hipMemcpy(dEin, hE, nE * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dCin, hC, nC * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dt, ht, (size_t)N * 8, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(ddl, hdl, (size_t)N * 4, hipMemcpyHostToDevice));

  CCE_OK_(cce_forward(dEin, dCin, dt, N, V, D, CCE_BF16, ii, dloss, dlse, dtm, dws_f, fws, NULL,
                      st));
  CCE_OK_(cce_backward(ddl, 1, dEin, dCin, dt, dlse, dtm, N, V, D, CCE_BF16, ii, eps, 0.0f, ddE,
                       ddC, CCE_F32, dws_b, bws, dstats, st));
  HIP_OK(hipStreamSynchronize(st));

  float* hloss = malloc((size_t)N * 4);
  float* hlse = malloc((size_t)N * 4);
  float* hdE = malloc(nE * 4);
  float* hdC = malloc(nC * 4);
  int64_t hstats[2];
  if (!hloss || !hlse || !hdE || !hdC) {
    fprintf(stderr, "out of host memory\n");
    return 1;
  }
  HIP_OK(hipMemcpy(hloss, dloss, (size_t)N * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hlse, dlse, (size_t)N * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hdE, ddE, nE * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hdC, ddC, nC * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hstats, dstats, sizeof hstats, hipMemcpyDeviceToHost));

  FILE* out = fopen(argv[2], "wb");
  if (!out || !write_all(out, hloss, (size_t)N * 4) || !write_all(out, hlse, (size_t)N * 4) ||
      !write_all(out, hdE, nE * 4) || !write_all(out, hdC, nC * 4) ||
      !write_all(out, hstats, sizeof hstats)) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(out);

  void* bufs[] = {dEin, dCin, dt, ddl, dloss, dlse, dtm, dws_f, dws_b, ddE, ddC, dstats};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
  HIP_OK(hipStreamDestroy(st));
  free(hE);
  free(hC);
  free(ht);
  free(hdl);
  free(hloss);
  free(hlse);
  free(hdE);
  free(hdC);
  printf("cce_c_client: N=%lld V=%lld D=%lld skipped %lld of %lld blocks\n", (long long)N,
         (long long)V, (long long)D, (long long)hstats[0], (long long)hstats[1]);
  return 0;
}
