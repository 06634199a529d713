/* A C caller of libhc (no C++, no Python): checks that include/hc.h serves a
 * C99 program and that the entry points work through plain pointers.
 *
 *   hc_client abi   status strings, size queries and argument validation
 *                   (no device needed)
 *   hc_client gpu   on the current HIP device: hc_post with post = 0 and
 *                   comb = I returns the streams unchanged, hc_pre with a
 *                   one-hot pre returns that stream, and hc_boundary as the
 *                   stack exit (no projection) does both in one call -- all
 *                   bit for bit ("Write the streams" equation, Block.hc_pre).
 * Exit status 0 on success; the first failure is printed. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "hc.h"

#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      fprintf(stderr, "hc_client: " __VA_ARGS__);          \
      fprintf(stderr, " (%s)\n", hc_last_error());         \
      return 1;                                            \
    }                                                      \
  } while (0)
#define HIPCHECK(call) CHECK((call) == hipSuccess, "%s failed", #call)

static int abi(void) {
  CHECK(hc_version() >= 100, "hc_version");
  CHECK(strcmp(hc_strerror(HC_OK), "success") == 0, "hc_strerror");
  CHECK(hc_fn_packed_bytes(4, 5120) > 0 && hc_fn_packed_bytes(3, 5120) == 0, "hc_fn_packed_bytes");
  CHECK(hc_workspace_bytes(4096, 4, 5120) > 0 && hc_workspace_bytes(0, 4, 5120) == 0, "hc_workspace_bytes");
  CHECK(hc_pre(NULL, NULL, 16, 4, 64, NULL, NULL) == HC_EINVAL, "hc_pre(NULL) must be HC_EINVAL");
  CHECK(hc_post((const hc_bf16*)16, (const hc_bf16*)16, (const float*)16, (const float*)16, 16, 5, 64,
                (hc_bf16*)32, NULL) == HC_ENOTSUP, "hc_post(hc=5) must be HC_ENOTSUP");
  hc_boundary_args a;
  memset(&a, 0, sizeof a);
  a.struct_size = 4;
  CHECK(hc_boundary(&a, NULL) == HC_EINVAL, "hc_boundary(short struct) must be HC_EINVAL");
  printf("hc_client abi: ok (libhc %d)\n", hc_version());
  return 0;
}

static int gpu(void) {
  enum { N = 37, HC = 4, D = 1088 };
  const size_t nx = (size_t)N * HC * D, nd = (size_t)N * D;
  hc_bf16* hx = malloc(nx * sizeof *hx);
  hc_bf16* hd = malloc(nd * sizeof *hd);
  hc_bf16* hxo = malloc(nx * sizeof *hxo);
  hc_bf16* hy = malloc(nd * sizeof *hy);
  float* post = calloc((size_t)N * HC, sizeof(float));
  float* comb = calloc((size_t)N * HC * HC, sizeof(float));
  float* pre = calloc((size_t)N * HC, sizeof(float));
  CHECK(hx && hd && hxo && hy && post && comb && pre, "out of host memory");
  unsigned s = 12345u;
  for (size_t i = 0; i < nx; ++i) {                 /* finite bf16 patterns: exponents 120..135 */
    s = s * 1664525u + 1013904223u;
    hx[i] = (hc_bf16)(((s >> 16) & 0x807Fu) | ((120u + ((s >> 8) & 15u)) << 7));
  }
  for (size_t i = 0; i < nd; ++i) hd[i] = hx[i] ^ 0x8000u;
  for (int t = 0; t < N; ++t) {
    for (int j = 0; j < HC; ++j) comb[(t * HC + j) * HC + j] = 1.0f;
    pre[t * HC + (t % HC)] = 1.0f;
  }
  void *dx, *dd, *dxo, *dy, *dpost, *dcomb, *dpre;
  HIPCHECK(hipMalloc(&dx, nx * 2));
  HIPCHECK(hipMalloc(&dd, nd * 2));
  HIPCHECK(hipMalloc(&dxo, nx * 2));
  HIPCHECK(hipMalloc(&dy, nd * 2));
  HIPCHECK(hipMalloc(&dpost, (size_t)N * HC * 4));
  HIPCHECK(hipMalloc(&dcomb, (size_t)N * HC * HC * 4));
  HIPCHECK(hipMalloc(&dpre, (size_t)N * HC * 4));
  HIPCHECK(hipMemcpy(dx, hx, nx * 2, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(dd, hd, nd * 2, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(dpost, post, (size_t)N * HC * 4, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(dcomb, comb, (size_t)N * HC * HC * 4, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(dpre, pre, (size_t)N * HC * 4, hipMemcpyHostToDevice));

  /* hc_post: post = 0, comb = I -> X */
  CHECK(hc_post(dd, dx, dpost, dcomb, N, HC, D, dxo, NULL) == HC_OK, "hc_post");
  HIPCHECK(hipMemcpy(hxo, dxo, nx * 2, hipMemcpyDeviceToHost));
  CHECK(memcmp(hxo, hx, nx * 2) == 0, "hc_post with post = 0, comb = I changed the streams");
  /* hc_pre: one-hot pre -> that stream */
  CHECK(hc_pre(dx, dpre, N, HC, D, dy, NULL) == HC_OK, "hc_pre");
  HIPCHECK(hipMemcpy(hy, dy, nd * 2, hipMemcpyDeviceToHost));
  for (int t = 0; t < N; ++t)
    CHECK(memcmp(hy + (size_t)t * D, hx + ((size_t)t * HC + t % HC) * D, D * 2) == 0,
          "hc_pre with a one-hot pre is not the stream (token %d)", t);
  /* hc_boundary as the stack exit: both at once */
  HIPCHECK(hipMemset(dxo, 0, nx * 2));
  HIPCHECK(hipMemset(dy, 0, nd * 2));
  hc_boundary_args a;
  memset(&a, 0, sizeof a);
  a.struct_size = sizeof a;
  a.hc = HC; a.d = D; a.n = N; a.iters = 20;
  a.hc_eps = 1e-6f; a.norm_eps = 1e-6f; a.rms_eps = 1e-6f;
  a.delta = dd; a.x = dx; a.post_in = dpost; a.comb_in = dcomb; a.pre_in = dpre;
  a.x_out = dxo; a.y_out = dy;
  CHECK(hc_boundary(&a, NULL) == HC_OK, "hc_boundary");
  HIPCHECK(hipDeviceSynchronize());
  HIPCHECK(hipMemcpy(hxo, dxo, nx * 2, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(hy, dy, nd * 2, hipMemcpyDeviceToHost));
  CHECK(memcmp(hxo, hx, nx * 2) == 0, "hc_boundary exit: x_out differs from the streams");
  for (int t = 0; t < N; ++t)
    CHECK(memcmp(hy + (size_t)t * D, hx + ((size_t)t * HC + t % HC) * D, D * 2) == 0,
          "hc_boundary exit: y is not the one-hot stream (token %d)", t);
  hipFree(dx); hipFree(dd); hipFree(dxo); hipFree(dy); hipFree(dpost); hipFree(dcomb); hipFree(dpre);
  free(hx); free(hd); free(hxo); free(hy); free(post); free(comb); free(pre);
  printf("hc_client gpu: ok\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "abi") == 0) return abi();
  if (argc == 2 && strcmp(argv[1], "gpu") == 0) return abi() || gpu();
  fprintf(stderr, "usage: hc_client abi|gpu\n");
  return 2;
}
